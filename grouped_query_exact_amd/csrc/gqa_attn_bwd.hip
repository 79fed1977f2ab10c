// Backward pass of exact grouped-query attention for gfx950 (MI355X).
//
// With P = softmax(scale * Q K^T) (recomputed from Q, K and the forward's
// log-sum-exp), O the forward output and dO the upstream gradient:
//   D_i  = sum_c dO[i,c] O[i,c]
//   dS   = P * (dO V^T - D)
//   dQ   = scale * dS K
//   dK   = scale * dS^T Q   and   dV = P^T dO,  both summed over the G query
//          heads of a KV group (the heads share K and V)
// The pages benchmark the forward and backward passes together
// (batch-sensitivity article, "performance analysis"); the gradients are the
// chain rule of the forward definition.
//
// Two kernels, both on PackGQA rows (row r of a KV group is token r / G,
// query head g*G + r % G):
//  * bwd_dq_kernel: the forward kernel's tiling (128 rows, 64-key tiles
//    through a double-buffered LDS ring): S^T = K Q^T and dP^T = V dO^T with
//    Q and dO rows in registers, dS in registers as the B operand of
//    dQ^T += K^T dS^T, K^T read with the transposing LDS read. It also
//    forms D of its rows and stores D and -LSE*log2(e) for the next kernel.
//  * bwd_dkdv_kernel: 128 keys per workgroup of eight wavefronts, a pair per
//    32 keys: the dV wave holds the keys' K rows in registers, forms S and P
//    and hands P to the dK wave (V rows in registers) through LDS one tile
//    later. The workgroup streams every query tile (64 packed rows of Q and
//    dO, last tile first) of the KV group through a ring of LDS stages, so
//    dK and dV collect all G heads without atomics. S = Q K^T and
//    dP = dO V^T come out of the matrix cores with one key per lane, which
//    is already the A-operand layout of dV += P^T dO and dK += dS^T Q; dO
//    and Q enter those products through the transposing LDS read, with their
//    rows read in the order the score registers hold them.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace gqa {

// 4-byte global -> LDS copy of every lane: lane l writes LDS bytes
// [lds + 4*l, lds + 4*l + 4) with the 4 bytes at base + voff (the kernel
// waits for it with vmcnt before the barrier that publishes the tile).
__device__ __forceinline__ void lds_dma4(const void* base, uint32_t voff, LDS void* lds) {
    const uint32_t m0 = (uint32_t)(size_t)lds;
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2"
                 :
                 : "s"(m0), "v"(voff), "s"(base)
                 : "memory", "m0");
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// log2-domain log-sum-exp of a row; a row without visible keys (LSE = -inf)
// gets +inf so that exp2(-inf - (+inf)) = 0 for all of its (masked) scores.
__device__ __forceinline__ float lse2_of(float lse) {
    return lse == -__builtin_inff() ? __builtin_inff() : lse * kLog2e;
}

// ---------------------------------------------------------------- dQ
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dq_kernel(const BwdParams p) {
    constexpr int TILE_B = kBlockN * D * 2;
    constexpr int NCH = D / 8;
    constexpr int NLOAD = kBlockN * NCH / kThreads;
    __shared__ __attribute__((aligned(16))) uint16_t smem[4 * kBlockN * D];
    LDS char* lds = (LDS char*)smem;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int col = lane & 31, half = lane >> 5;

    const int logical = xcd_remap(blockIdx.x, p.grid_dq);
    const int rt = p.row_tiles - 1 - (logical % p.row_tiles);  // heaviest causal tiles first
    const int tmp = logical / p.row_tiles;
    const int g = tmp % p.Hk;
    const int b = tmp / p.Hk;
    const int h0 = g * p.G;
    const int r0 = rt * kBlockM;

    const int r = r0 + wave * 32 + col;
    const bool row_valid = r < p.R;
    const int rc = min(r, p.R - 1);
    const int ti = (int)fdiv((uint32_t)rc, p.gmul, p.gshift);
    const int hh = h0 + (rc - ti * p.G);
    const int koff = p.Sk - p.Sq;

    // Q and dO rows -> registers (B operands of S^T = K Q^T and dP^T = V dO^T).
    // Every packed row belongs to exactly one workgroup, which also forms its
    // D = sum(dO * O) (lanes l and l+32 hold the two halves of the row) and
    // stores D and -LSE*log2(e) for the dK/dV kernel that runs next.
    bf16x8 qreg[D / 16], oreg[D / 16];
    float dpart = 0.f;
    {
        const int64_t grow = ((int64_t)b * p.Sq + ti) * p.Hq + hh;
        const uint16_t* qrow = p.q + grow * D;
        const uint16_t* grow_p = p.dout + grow * D;
        const uint16_t* orow = p.o + grow * D;
#pragma unroll
        for (int dc = 0; dc < D / 16; ++dc) {
            qreg[dc] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qrow + dc * 16 + half * 8));
            const u32x4 gv = *(const u32x4*)(grow_p + dc * 16 + half * 8);
            const u32x4 ov = *(const u32x4*)(orow + dc * 16 + half * 8);
            oreg[dc] = __builtin_bit_cast(bf16x8, gv);
#pragma unroll
            for (int j = 0; j < 4; ++j) dpart += bf16_lo(gv[j]) * bf16_lo(ov[j]) + bf16_hi(gv[j]) * bf16_hi(ov[j]);
        }
    }
    const float drow = xhalf_sum(dpart);
    const int64_t lrow = ((int64_t)b * p.Hq + hh) * p.Sq + ti;
    const float lse2 = lse2_of(p.lse[lrow]);
    if (row_valid && half == 0) {
        p.drow[lrow] = drow;
        p.nlse2[lrow] = -lse2;
    }

    const int r_last = min(r0 + kBlockM, p.R) - 1;
    const int i_max = (int)fdiv((uint32_t)r_last, p.gmul, p.gshift);
    int kv_end = p.Sk;
    if (CAUSAL) kv_end = min(p.Sk, i_max + koff + 1);
    const int T = kv_end > 0 ? (kv_end + kBlockN - 1) / kBlockN : 0;

    const int rw0 = r0 + wave * 32;
    const bool wave_active = rw0 < p.R;
    const int iw_min = (int)fdiv((uint32_t)min(rw0, p.R - 1), p.gmul, p.gshift);
    const int iw_max = (int)fdiv((uint32_t)(min(rw0 + 32, p.R) - 1), p.gmul, p.gshift);

    const int64_t kv_stride_b = (int64_t)p.Hk * D * 2;
    const char* kbase = (const char*)(p.k + ((int64_t)b * p.Sk * p.Hk + g) * D);
    const char* vbase = (const char*)(p.v + ((int64_t)b * p.Sk * p.Hk + g) * D);
    uint32_t goff[NLOAD];
#pragma unroll
    for (int u = 0; u < NLOAD; ++u) {
        const int ci = (u * 4 + wave) * 64 + lane;
        const int row = ci / NCH;
        goff[u] = (uint32_t)(row * kv_stride_b + (((ci % NCH) ^ swz<D>(row)) * 16));
    }
    auto issue = [&](int kv0, int buf) {
        LDS char* kt = lds + buf * 2 * TILE_B;
        LDS char* vt = kt + TILE_B;
        const char* kg = kbase + kv0 * kv_stride_b;
        const char* vg = vbase + kv0 * kv_stride_b;
        if (kv0 + kBlockN <= p.Sk) {
#pragma unroll
            for (int u = 0; u < NLOAD; ++u) {
                const int dst = (u * 4 + wave) * 1024;
                lds_dma16(kg, goff[u], kt + dst);
                lds_dma16(vg, goff[u], vt + dst);
            }
        } else {  // ragged last tile: rows past the end re-read the last key (masked)
#pragma unroll
            for (int u = 0; u < NLOAD; ++u) {
                const int dst = (u * 4 + wave) * 1024;
                const int ci = (u * 4 + wave) * 64 + lane;
                const int row = ci / NCH;
                const int key = min(kv0 + row, p.Sk - 1) - kv0;
                const uint32_t o = (uint32_t)(key * kv_stride_b + (((ci % NCH) ^ swz<D>(row)) * 16));
                lds_dma16(kg, o, kt + dst);
                lds_dma16(vg, o, vt + dst);
            }
        }
    };

    // A operands read as in the forward kernel: K (and V) rows in the key
    // order pi32 for S^T / dP^T, K^T through the transposing read for dQ^T.
    const int krow0 = pi32(col);
    uint32_t kofs[D / 16];
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc) kofs[dc] = krow0 * (D * 2) + (((2 * dc + half) ^ swz<D>(krow0)) * 16);
    const int u16 = lane & 15, qq = (lane >> 4) & 1;
    const int rho = ((u16 & 1) << 1) | ((u16 >> 1) & 1);
    uint32_t tofs[D / 32][2];
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
            const int trow = half * 8 + rr * 4 + (u16 >> 2);
            const int tcol = cb * 32 + qq * 16 + rho * 4;
            tofs[cb][rr] = trow * (D * 2) + (((tcol >> 3) ^ swz<D>(trow)) * 16) + (tcol & 7) * 2;
        }

    f32x16 acc[D / 32];
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) acc[cb] = f32x16{};
    const float c = p.c;
    const int jlim = CAUSAL ? min(p.Sk - 1, ti + koff) : p.Sk - 1;

    auto compute = [&](int buf, int kv0, bool need_mask) {
        const LDS char* kt = lds + buf * 2 * TILE_B;
        const LDS char* vt = kt + TILE_B;
        f32x16 sacc[2], pacc[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            sacc[mb] = f32x16{};
            pacc[mb] = f32x16{};
#pragma unroll
            for (int dc = 0; dc < D / 16; ++dc) {
                const bf16x8 ak = *(const LDS bf16x8*)(kt + kofs[dc] + mb * 32 * D * 2);
                sacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, qreg[dc], sacc[mb], 0, 0, 0);
                const bf16x8 av = *(const LDS bf16x8*)(vt + kofs[dc] + mb * 32 * D * 2);
                pacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, oreg[dc], pacc[mb], 0, 0, 0);
            }
        }
        // dS = P (dP - D), P = exp2(s c - lse2); slot i of this lane holds key
        // kv0 + 32*mb + 16*(i/8) + 8*half + (i%8)
        const int lim = jlim - kv0 - half * 8;
        bf16x8 ds[4];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float x = __builtin_fmaf(sacc[mb][i], c, -lse2);
                if (need_mask && mb * 32 + ((i >> 3) << 4) + (i & 7) > lim) x = -__builtin_inff();
                const float pv = __builtin_amdgcn_exp2f(x);
                ds[mb * 2 + (i >> 3)][i & 7] = (__bf16)(pv * (pacc[mb][i] - drow));
            }
        // dQ^T += K^T dS^T
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
            for (int cb = 0; cb < D / 32; ++cb) {
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS s16x4*)(kt + tofs[cb][0] + kk * 16 * D * 2));
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS s16x4*)(kt + tofs[cb][1] + kk * 16 * D * 2));
                const s16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), ds[kk], acc[cb], 0, 0, 0);
            }
        }
    };

    if (T > 0) issue(0, 0);
    for (int t = 0; t < T; ++t) {
        const int buf = t & 1;
        wait_vmem();
        __syncthreads();
        if (t + 1 < T) issue((t + 1) * kBlockN, buf ^ 1);
        const int kv0 = t * kBlockN;
        if (wave_active && !(CAUSAL && kv0 > iw_max + koff)) {
            const bool need_mask = (kv0 + kBlockN > p.Sk) || (CAUSAL && kv0 + kBlockN - 1 > iw_min + koff);
            compute(buf, kv0, need_mask);
        }
    }

    if (row_valid) {
        uint16_t* drow_out = p.dq + (((int64_t)b * p.Sq + ti) * p.Hq + hh) * D;
        const float sc = p.scale;
#pragma unroll
        for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
            for (int run = 0; run < 2; ++run) {
                bf16x8 ov;
#pragma unroll
                for (int i = 0; i < 8; ++i) ov[i] = (__bf16)(acc[cb][run * 8 + i] * sc);
                *(bf16x8*)(drow_out + cb * 32 + run * 16 + half * 8) = ov;
            }
    }
}

// ---------------------------------------------------------------- dK, dV
// Eight wavefronts over 128 keys, 32 keys per pair of wavefronts w and w+4
// (which share a SIMD): wave w+4 computes S = Q K^T and P for query tile j,
// adds P^T dO to dV and hands P (bf16, the operand it used) to wave w
// through LDS; one tile later wave w forms dP = dO V^T, dS = P (dP - D) and
// adds dS^T Q to dK. Each wave issues 8 matrix products per 16 query rows,
// holds one accumulator, and has room for the second wavefront on its SIMD
// to hide its latencies. The two kinds run separate copies of the tile loop
// with the same barriers; a tile of BM rows is MB blocks of 32.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dkdv_kernel(const BwdParams p) {
    constexpr int BM = kBwdRows;                      // packed query rows per tile
    constexpr int MB = BM / 32;                       // 32-row blocks per tile
    static_assert(BM == 32 || BM == 64, "32 or 64 rows per tile");
    constexpr int NCH = D / 8;                        // 16-byte chunks per row
    constexpr int TILE_B = BM * D * 2;                // bytes of a Q or dO tile
    constexpr int NCOPY = 2 * BM * NCH / kBwdThreads; // 16-byte copies per thread and tile (Q and dO)
    static_assert(NCOPY >= 1 && (BM * NCH) % 64 == 0, "a wave's copies stay inside one tensor");
    constexpr int STAGE_B = 2 * TILE_B + 2 * 64 * 4;  // Q, dO, 64 -LSE*log2(e) and 64 D slots
    constexpr int STAGES = kBwdStages;
    static_assert(STAGES >= 3, "tiles j-1 and j are in use while j+STAGES-2 is copied");
    constexpr int PAIR_PB = MB * 2 * 64 * 16;         // bf16 P of one tile for one pair
    // copies per wave and tile: its Q / dO chunks, plus the LSE / D row for waves 0 and 1
    constexpr int COPIES_LO = NCOPY + 1, COPIES_HI = NCOPY;
    static_assert(COPIES_LO * (STAGES - 3) < 64, "vmcnt is a 6-bit field");
    __shared__ __attribute__((aligned(16))) char smem_raw[STAGES * STAGE_B + 2 * 4 * PAIR_PB];
    LDS char* lds = (LDS char*)smem_raw;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int col = lane & 31, half = lane >> 5;

    const int logical = xcd_remap(blockIdx.x, p.grid_dkdv);
    const int kb = logical % p.key_blocks;           // key blocks of one (b, g) adjacent: they share Q, dO
    const int tmp = logical / p.key_blocks;
    const int g = tmp % p.Hk;
    const int b = tmp / p.Hk;
    const int k0 = kb * kBwdKeys;
    const int pair = wave & 3;
    const int kw0 = k0 + pair * 32;                  // this pair's keys kw0 .. kw0+31
    const int key = kw0 + col;                       // this lane's key (column of S)
    const int keyc = min(key, p.Sk - 1);
    const int koff = p.Sk - p.Sq;

    // query tiles: from the first row whose token sees key k0 (causal) to the end
    int tile_begin = 0;
    if (CAUSAL) tile_begin = (int)(((int64_t)max(0, k0 - koff) * p.G) / BM);
    const int tile_end = (p.R + BM - 1) / BM;
    const int n = max(0, tile_end - tile_begin);
    // The j-th tile of the loop, last tile first: the key blocks of a KV
    // group start together, so each Q / dO tile is read by all of them at
    // about the same time and leaves HBM once (in ascending order, where
    // block kb starts 128 keys' worth of tokens later, the group's 4 MB of Q
    // and dO went through the L2 several times: 0.92 GB instead of 0.19 GB
    // per call at the Llama-2 shape).
    auto tile_of = [&](int j) { return tile_end - 1 - j; };

    // Tile copies: packed row -> (token, head) -> [B, Sq, Hq, D] offset. The
    // Q and dO chunks of a tile are numbered 0 .. 2*BM*NCH-1 (Q first) and
    // chunk cc lands at byte 16*cc of the stage; a wave's 64 chunks belong to
    // one tensor. Wave 0 copies the rows' -LSE*log2(e), wave 1 their D
    // (with 32-row tiles lanes 32..63 repeat rows 0..31).
    const char* qb = (const char*)(p.q + (int64_t)b * p.Sq * p.Hq * D);
    const char* ob = (const char*)(p.dout + (int64_t)b * p.Sq * p.Hq * D);
    const char* lb = (const char*)(wave == 0 ? p.nlse2 : p.drow) + (int64_t)b * p.Hq * p.Sq * 4;
    auto chunk_offset = [&](int r0, int u, int& cw) {  // byte offset of this lane's chunk u of tile rows r0..
        cw = (u * (kBwdThreads / 64) + wave) * 64;
        const int ci = cw - (cw >= BM * NCH ? BM * NCH : 0) + lane;
        const int row = ci / NCH;
        const int rr = min(r0 + row, p.R - 1);
        const int tok = (int)fdiv((uint32_t)rr, p.gmul, p.gshift);
        const int head = g * p.G + (rr - tok * p.G);
        return (uint32_t)((((int64_t)tok * p.Hq + head) * D + (((ci % NCH) ^ swz<D>(row)) * 8)) * 2);
    };
    auto row_offset = [&](int r0) {
        const int rr = min(r0 + (lane & (BM - 1)), p.R - 1);
        const int tok = (int)fdiv((uint32_t)rr, p.gmul, p.gshift);
        const int head = g * p.G + (rr - tok * p.G);
        return (uint32_t)(((int64_t)head * p.Sq + tok) * 4);
    };
    // When G divides the tile height, tile t holds the rows of tile 0 moved by
    // t*BM/G tokens: its copies use tile 0's offsets and a scalar base step.
    const bool shifted = (BM % p.G) == 0;
    const int64_t qstep = shifted ? (int64_t)(BM / p.G) * p.Hq * D * 2 : 0;
    const int64_t lstep = shifted ? (int64_t)(BM / p.G) * 4 : 0;
    uint32_t off0[NCOPY];
#pragma unroll
    for (int u = 0; u < NCOPY; ++u) {
        int cw;
        off0[u] = chunk_offset(0, u, cw);
    }
    const uint32_t loff0 = row_offset(0);
    auto issue = [&](int tile, int stage) {
        LDS char* st = lds + stage * STAGE_B;
        const int r0 = tile * BM;
        if (shifted && r0 + BM <= p.R) {
#pragma unroll
            for (int u = 0; u < NCOPY; ++u) {
                const int cw = (u * (kBwdThreads / 64) + wave) * 64;
                lds_dma16((cw >= BM * NCH ? ob : qb) + tile * qstep, off0[u], st + cw * 16);
            }
            if (wave < 2) lds_dma4(lb + tile * lstep, loff0, st + 2 * TILE_B + wave * 256);
        } else {  // G does not divide the tile, or the ragged last tile (rows clamped)
#pragma unroll
            for (int u = 0; u < NCOPY; ++u) {
                int cw;
                const uint32_t off = chunk_offset(r0, u, cw);
                lds_dma16(cw >= BM * NCH ? ob : qb, off, st + cw * 16);
            }
            if (wave < 2) lds_dma4(lb, row_offset(r0), st + 2 * TILE_B + wave * 256);
        }
    };

    // A operand (S = Q K^T, dP = dO V^T): row 32*mb + col of the tile, d
    // chunk 2*dc + half (the swizzle repeats every 16 rows)
    uint32_t aofs[D / 16];
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc) aofs[dc] = col * (D * 2) + (((2 * dc + half) ^ swz<D>(col)) * 16);
    // B operand of dV += P^T dO and dK += dS^T Q (transposing read): for the
    // 16-row block kb2, read rr, lane u16 of its 16-lane group addresses row
    // 16*kb2 + 8*rr + 4*half + u16/4, columns 32*cb + 16*qq + 4*(u16%4); the
    // read hands lane t column 32*cb + 16*qq + t of the rows that slots
    // 8*(kb2%2) + 4*rr .. +3 of the score registers of block kb2/2 hold.
    const int u16 = lane & 15, qq = (lane >> 4) & 1;
    uint32_t bofs[D / 32][2];
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
            const int brow = rr * 8 + half * 4 + (u16 >> 2);   // + 16*kb2 keeps the swizzle
            const int bcol = cb * 32 + qq * 16 + (u16 & 3) * 4;
            bofs[cb][rr] = brow * (D * 2) + (((bcol >> 3) ^ swz<D>(brow)) * 16) + (bcol & 7) * 2;
        }
    // P hand-over: the bf16 A operand of block mb, slot h (registers 8h .. 8h+7)
    // of lane l at 1024*(2*mb + h) + 16*l of the pair's area, two tiles' worth
    // (by tile parity)
    LDS char* pslot = lds + STAGES * STAGE_B + pair * PAIR_PB + lane * 16;
    const float c = p.c;

    // The tile loop of one kind of wave (DK: dK, else dV). Iteration j: the
    // dV waves compute tile j, the dK waves tile j-1 (whose P the barrier of
    // iteration j publishes). Tile j+STAGES-2 is copied into the stage of
    // tile j-2, which no wave uses after that barrier.
    auto run = [&](auto dk_tag) {
        constexpr bool DK = decltype(dk_tag)::value;
#pragma unroll
        for (int j = 0; j < STAGES - 2; ++j)
            if (j < n) issue(tile_of(j), j);

        // K (dV waves) or V (dK waves) rows of the pair's keys -> registers
        // (B operand of S = Q K^T or dP = dO V^T), loaded after the first
        // tiles' copies so that one latency covers both. The empty asm makes
        // the compiler wait for these loads here, once, rather than at their
        // first use inside the loop, where its wait would also drain the
        // copies in flight.
        bf16x8 breg[D / 16];
        {
            const uint16_t* src = (DK ? p.v : p.k) + (((int64_t)b * p.Sk + keyc) * p.Hk + g) * D;
#pragma unroll
            for (int dc = 0; dc < D / 16; ++dc)
                breg[dc] = __builtin_bit_cast(bf16x8, *(const u32x4*)(src + dc * 16 + half * 8));
#pragma unroll
            for (int dc = 0; dc < D / 16; ++dc) asm volatile("" ::"v"(breg[dc]));
        }

        f32x16 acc[D / 32];  // dK (unscaled) or dV
#pragma unroll
        for (int cb = 0; cb < D / 32; ++cb) acc[cb] = f32x16{};

        for (int j = 0; j <= n; ++j) {
            if (j < n) {  // copies complete in issue order: leave the later tiles' in flight
                if (j + STAGES - 3 < n) {
                    if (wave < 2) wait_vmem_n<COPIES_LO * (STAGES - 3)>();
                    else wait_vmem_n<COPIES_HI * (STAGES - 3)>();
                } else {
                    wait_vmem();
                }
            }
            __syncthreads();
            if (j + STAGES - 2 < n) issue(tile_of(j + STAGES - 2), (j + STAGES - 2) % STAGES);
            const int jt = DK ? j - 1 : j;
            if (jt < 0 || jt >= n) continue;
            const int r0 = tile_of(jt) * BM;
            // tokens of the tile; a pair computes only if one of its keys is visible
            const int tok_min = (int)fdiv((uint32_t)r0, p.gmul, p.gshift);
            const int tok_max = (int)fdiv((uint32_t)(min(r0 + BM, p.R) - 1), p.gmul, p.gshift);
            if (kw0 >= p.Sk || (CAUSAL && kw0 > tok_max + koff)) continue;
            const LDS char* qt = lds + (jt % STAGES) * STAGE_B;
            const LDS char* ot = qt + TILE_B;
            const LDS float* lt = (const LDS float*)(qt + 2 * TILE_B);
            LDS char* ps = pslot + (jt & 1) * (4 * PAIR_PB);
            const bool need_mask = !DK && ((r0 + BM > p.R) || (kw0 + 32 > p.Sk) || (CAUSAL && kw0 + 31 > tok_min + koff));
            bf16x8 a[2 * MB];  // dV: P, dK: dS (bf16 A operands), slot i of block mb in a[2*mb + i/8][i%8]
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                // S = Q K^T (dV) or dP = dO V^T (dK) of rows 32*mb..; register i
                // holds row 32*mb + 8*(i/4) + 4*half + (i%4) and key `key`
                f32x16 s = f32x16{};
#pragma unroll
                for (int dc = 0; dc < D / 16; ++dc) {
                    const bf16x8 x = *(const LDS bf16x8*)((DK ? ot : qt) + mb * 32 * D * 2 + aofs[dc]);
                    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, breg[dc], s, 0, 0, 0);
                }
                if (!DK) {
                    float x[16];
#pragma unroll
                    for (int j4 = 0; j4 < 4; ++j4) {
                        const f32x4 l4 = *(const LDS f32x4*)(lt + 32 * mb + 8 * j4 + 4 * half);
#pragma unroll
                        for (int e = 0; e < 4; ++e) x[4 * j4 + e] = __builtin_fmaf(s[4 * j4 + e], c, l4[e]);
                    }
                    if (need_mask) {
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const int rr = r0 + 32 * mb + 8 * (i >> 2) + 4 * half + (i & 3);
                            const int tok = (int)fdiv((uint32_t)min(rr, p.R - 1), p.gmul, p.gshift);
                            if (rr >= p.R || key >= p.Sk || (CAUSAL && key > tok + koff)) x[i] = -__builtin_inff();
                        }
                    }
#pragma unroll
                    for (int i = 0; i < 16; ++i) a[2 * mb + (i >> 3)][i & 7] = (__bf16)__builtin_amdgcn_exp2f(x[i]);
#pragma unroll
                    for (int h = 0; h < 2; ++h) *(LDS bf16x8*)(ps + (2 * mb + h) * 1024) = a[2 * mb + h];
                } else {
                    const LDS float* dt = lt + 64 + 32 * mb;
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const bf16x8 pv = *(const LDS bf16x8*)(ps + (2 * mb + h) * 1024);
#pragma unroll
                        for (int j4 = 0; j4 < 2; ++j4) {
                            const f32x4 d4 = *(const LDS f32x4*)(dt + 8 * (2 * h + j4) + 4 * half);
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const int i = 8 * h + 4 * j4 + e;
                                a[2 * mb + h][i & 7] = (__bf16)((float)pv[i & 7] * (s[i] - d4[e]));
                            }
                        }
                    }
                }
            }
            // dV += P^T dO or dK += dS^T Q, the second factor read transposed
            const LDS char* xt = DK ? qt : ot;
#pragma unroll
            for (int kb2 = 0; kb2 < 2 * MB; ++kb2) {
#pragma unroll
                for (int cb = 0; cb < D / 32; ++cb) {
                    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS s16x4*)(xt + bofs[cb][0] + kb2 * 16 * D * 2));
                    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS s16x4*)(xt + bofs[cb][1] + kb2 * 16 * D * 2));
                    const s16x8 bx = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                    acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kb2], __builtin_bit_cast(bf16x8, bx), acc[cb], 0, 0, 0);
                }
            }
        }

        // dK = scale * acc, dV = acc: lane holds column 32*cb + col of keys kw0 + 8*(i/4) + 4*half + (i%4)
        const float sc = DK ? p.scale : 1.0f;
        uint16_t* dst = DK ? p.dk : p.dv;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int kk = kw0 + 8 * (i >> 2) + 4 * half + (i & 3);
            if (kk < p.Sk) {
                const int64_t krow = (((int64_t)b * p.Sk + kk) * p.Hk + g) * D;
#pragma unroll
                for (int cb = 0; cb < D / 32; ++cb)
                    dst[krow + cb * 32 + col] = __builtin_bit_cast(uint16_t, (__bf16)(acc[cb][i] * sc));
            }
        }
    };
    if (wave < 4) run(std::true_type{});
    else run(std::false_type{});
}

// ---------------------------------------------------------------- launcher
// Sq == 0: only dK = dV = 0 is written (by the dK/dV kernel, which then has
// no query tile). The caller rejects Sk == 0 with queries.
template <int D, bool CAUSAL>
static hipError_t launch_bwd_d(const BwdParams& p, hipStream_t stream) {
    if ((int64_t)p.B * p.Sq * p.Hq > 0) {
        hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3(p.grid_dq), dim3(kThreads), 0, stream, p);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (p.grid_dkdv > 0)
        hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3(p.grid_dkdv), dim3(kBwdThreads), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_backward(const BwdParams& p, int d, bool causal, hipStream_t stream) {
    if (d == 128) return causal ? launch_bwd_d<128, true>(p, stream) : launch_bwd_d<128, false>(p, stream);
    return causal ? launch_bwd_d<64, true>(p, stream) : launch_bwd_d<64, false>(p, stream);
}

}  // namespace gqa
