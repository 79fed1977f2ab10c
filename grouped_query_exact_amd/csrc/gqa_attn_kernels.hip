// Grouped-query attention forward kernels for gfx950 (MI355X).
//
// The attention kernel computes, for one tile of 128 query rows against the
// keys of one KV head, the exact result of softmax(scale * Q K^T) V with a
// tiled online softmax (running row maximum and sum) and emits the natural
// log-sum-exp of every row. Query head h reads KV head h / (Hq/Hk)
// (batch-sensitivity article, "core design of grouped-query attention").
// With PackGQA (batch-sensitivity article, "Flash-Attention's PackGQA
// optimisation"; rise-and-fall tuning article, "root cause") the rows of a
// tile are the G query heads of one KV group, token-major: packed row r is
// token r / G, head g*G + r % G. With split-KV ("split + combine",
// rise-and-fall tuning article, "fix" table) a workgroup handles one part of
// the tile's keys and writes a normalised fp32 partial and its log-sum-exp;
// the combine kernel merges the parts with weights exp(LSE_s - LSE).
//
// Mapping onto CDNA4:
//  * 256 threads = 4 wavefronts; wave w owns rows [32w, 32w+32) of the tile.
//    Lane l owns row (l % 32); lanes l and l+32 share a row and split its
//    keys (for scores) and its head-dimension columns (for the output).
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: the A operand is 32 keys read from LDS, the
//    B operand is the wave's 32 query rows held in registers for the whole
//    key loop. Each lane then holds 32 scores of its own row, so the row
//    maximum is 31 in-lane max operations plus one exchange with lane l^32.
//  * The output is accumulated transposed, O^T += V^T P^T, with the same
//    MFMA: P^T (bf16) comes straight from the score registers, V^T is read
//    from a natural-layout V tile in LDS with ds_read_b64_tr_b16.
//  * K and V tiles travel HBM -> LDS with 16-byte global_load_lds (no VGPR
//    staging), double-buffered so the next tile streams in during compute.
//    LDS rows are stored with an XOR swizzle of their 16-byte chunks so the
//    MFMA operand reads are free of bank conflicts.
//  * Rows of 32 keys are stored in LDS in the order pi (below) so the score
//    registers of a lane hold runs of 8 consecutive keys and the output
//    registers hold runs of 8 consecutive head-dimension columns.
//  * Online softmax in base 2 with scale*log2(e) folded into one FMA, and a
//    lazily updated integral row maximum, raised (and the accumulator
//    rescaled by an exact power of two) to an integer only when a row needs
//    it. The prefill kernels form a tile's probabilities against the maximum
//    as it stands and raise it only on a row's first visible key or when a
//    partial sum of the tile's probabilities exceeds 2^20 (softmax_exps), so
//    no per-tile row maximum is needed; the decode kernel raises when the
//    tile's row maximum exceeds the running one by more than 2^8 (raise_max).
//    Every row's final O = acc / l uses the same maximum for numerator and
//    denominator, so the result is the same exact softmax, and tilings that
//    meet other integral maxima round the same probabilities to bf16.
//  * Causal tiles above the diagonal are never loaded; waves whose rows see
//    none of a tile's keys skip its arithmetic; only boundary tiles evaluate
//    the mask.
//  * Workgroup ids are remapped so that consecutive work items (all row tiles
//    of one batch element and KV group, heaviest causal tiles first) land on
//    the same XCD and share its L2.
//  * With fp8 e4m3 Q and K (QK8) the scores run on the fp8 matrix cores
//    (32x32x64 products, 2 per 32 keys at d=128 instead of 8) from an fp8 K
//    tile; V, P V and everything after the scores are the bf16 path's.
// The decode kernel further down takes head units of at most 32 rows (one
// wavefront, a deeper ring, optional paged or fp8 K/V).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace gqa {

// Extent of sequence b of a variable-length (packed) call: query tokens
// [qtok0, qtok0 + Sq) of q, keys [ktok0, ktok0 + Sk) of k and v. The offsets
// are clamped into the packed tensors and Sq to the grid's max_seqlen_q, so
// no offsets make a read or a write leave the buffers. Scalar loads
// (constant address space): the values are wave-uniform.
__device__ __forceinline__ void seq_extent(const FwdParams& p, int b, int64_t& qtok0, int& Sq, int64_t& ktok0, int& Sk) {
    typedef const __attribute__((address_space(4))) int* cint_p;
    const cint_p cq = (cint_p)p.cu_q;
    const cint_p ck = (cint_p)p.cu_k;
    const int q0 = min(max(cq[b], 0), p.total_q);
    const int q1 = min(max(cq[b + 1], q0), p.total_q);
    const int k0 = min(max(ck[b], 0), p.total_k);
    const int k1 = min(max(ck[b + 1], k0), p.total_k);
    qtok0 = __builtin_amdgcn_readfirstlane(q0);
    Sq = __builtin_amdgcn_readfirstlane(min(q1 - q0, p.Sq));
    ktok0 = __builtin_amdgcn_readfirstlane(k0);
    Sk = __builtin_amdgcn_readfirstlane(k1 - k0);
}

// LSE element of (batch b, head hh, token ti): [B, Hq, Sq], or [Hq, total_q]
// for variable-length calls (token qtok0 + ti of the packed axis).
__device__ __forceinline__ int64_t lse_index(const FwdParams& p, int b, int hh, int64_t qtok0, int ti, bool varlen) {
    return varlen ? (int64_t)hh * p.total_q + qtok0 + ti : ((int64_t)b * p.Hq + hh) * p.Sq + ti;
}

// Row `row` of the split workspace ([B*Sq or total_q, Hq]) -> its LSE element.
__device__ __forceinline__ int64_t lse_row(const CombineParams& p, int64_t row) {
    const int64_t hq = row % p.Hq;
    const int64_t bt = row / p.Hq;
    return ((bt / p.Sq) * p.Hq + hq) * p.Sq + bt % p.Sq;
}

// Whether the attention kernel wrote the partials of workspace row `row`.
// Variable-length calls: token t = row / Hq belongs to the last sequence whose
// first token is <= t and was written iff it is among that sequence's first
// min(length, max_seqlen_q) tokens (offsets clamped as in seq_extent); tokens
// past the last sequence belong to none. Other calls write every row.
__device__ __forceinline__ bool row_written(const CombineParams& p, int64_t row) {
    if (!p.cu_q) return true;
    typedef const __attribute__((address_space(1))) int* gint_p;
    const gint_p cu = (gint_p)p.cu_q;
    const int t = (int)(row / p.Hq);
    int lo = 0, hi = p.B - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (min(max(cu[mid], 0), p.total_q) <= t) lo = mid;
        else hi = mid - 1;
    }
    const int q0 = min(max(cu[lo], 0), p.total_q);
    const int q1 = min(max(cu[lo + 1], q0), p.total_q);
    return t >= q0 && t - q0 < min(q1 - q0, p.max_sq);
}

// QK8: Q and K hold fp8 e4m3 bytes; S^T = K Q^T runs on the fp8 matrix
// cores (v_mfma_scale_f32_32x32x64_f8f6f4, unit block scales), V stays bf16.
template <int D, bool CAUSAL, bool SPLIT, bool VARLEN, bool QK8, bool PAGED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_fwd_kernel(const FwdParams p) {
    constexpr int TILE = kBlockN * D;                 // elements of one K or V tile
    constexpr int TILE_B = TILE * 2;                  // bytes (bf16; an fp8 K tile uses the first half)
    constexpr int NCH = D / 8;                        // 16-byte chunks per bf16 row
    constexpr int NLOAD = kBlockN * NCH / kThreads;   // 16-byte loads per thread per bf16 tensor
    constexpr int NCH8 = D / 16;                      // 16-byte chunks per fp8 row
    constexpr int NLOADK = QK8 ? kBlockN * NCH8 / kThreads : NLOAD;  // ... for the K tile
    __shared__ __attribute__((aligned(16))) uint16_t smem[4 * TILE];
    LDS char* lds = (LDS char*)smem;                  // [buf][K|V] tiles

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int col = lane & 31, half = lane >> 5;

    // ---- work item
    int s, rt, unit, b;
    if (!VARLEN) {
        const int logical = xcd_remap(blockIdx.x, p.grid);
        s = logical % p.ns;
        int tmp = logical / p.ns;
        rt = p.row_tiles - 1 - (tmp % p.row_tiles);  // heaviest causal tiles first
        tmp /= p.row_tiles;
        unit = tmp % p.units_per_b;
        b = tmp / p.units_per_b;
    } else if (p.worklist) {
        // sequences of very different lengths: the (sequence, row tile) pairs
        // that exist, heaviest first, from the scheduling kernel's work list
        // (scalar loads); the grid's spare workgroups past its end exit at once
        typedef const __attribute__((address_space(4))) int* cint_p;
        const cint_p wl = (cint_p)p.worklist;
        s = blockIdx.x % p.ns;
        const int tmp = blockIdx.x / p.ns;
        const int pair = tmp / p.units_per_b;
        unit = tmp % p.units_per_b;
        if (pair >= wl[0]) return;
        b = __builtin_amdgcn_readfirstlane(wl[1 + 2 * pair]);
        rt = __builtin_amdgcn_readfirstlane(wl[2 + 2 * pair]);
    } else {
        // sequences of about equal length: every row tile of the longest in
        // every sequence, the row tile the slowest index, so the heaviest
        // causal tiles of all sequences start first; items are not of equal
        // cost, so they are dealt round-robin over the XCDs
        s = blockIdx.x % p.ns;
        const int tmp = blockIdx.x / p.ns;
        const int nbu = p.B * p.units_per_b;
        rt = p.row_tiles - 1 - tmp / nbu;
        unit = (tmp % nbu) % p.units_per_b;
        b = (tmp % nbu) / p.units_per_b;
    }
    const int g = p.Gp > 1 ? unit : unit / p.G;   // KV head
    const int h0 = p.Gp > 1 ? unit * p.G : unit;  // first query head of the tile
    const int r0 = rt * kBlockM;

    // ---- this sequence: query tokens qtok0 .. qtok0+Sq-1, keys ktok0 .. ktok0+Sk-1
    int Sq = p.Sq, Sk = p.Sk;
    int64_t qtok0 = (int64_t)b * p.Sq, ktok0 = (int64_t)b * p.Sk;
    if (VARLEN) seq_extent(p, b, qtok0, Sq, ktok0, Sk);
    if (PAGED) Sk = __builtin_amdgcn_readfirstlane(min(max(p.seqlens_k[b], 0), p.max_pages * p.page_size));
    const int R = VARLEN ? Sq * p.Gp : p.R;  // rows of this head unit
    if (VARLEN && r0 >= R) return;            // row tile past the end of this sequence

    // ---- this lane's row: token ti, head hh
    const int r = r0 + wave * 32 + col;
    const bool row_valid = r < R;
    const int rc = min(r, R - 1);
    const int ti = (int)fdiv((uint32_t)rc, p.gmul, p.gshift);
    const int hh = h0 + (rc - ti * p.Gp);
    const int koff = Sk - Sq;  // bottom-right causal offset

    // ---- Q rows -> registers (B operand of S^T = K Q^T). fp8: operand t
    // covers d in [64t, 64t+64), lane half h holds bytes 64t+32h .. +31 (the
    // 32x32x64 product pairs byte j of a lane half of A with byte j of the
    // same lane half of B, so K is read with the same split).
    bf16x8 qreg[QK8 ? 1 : D / 16];
    i32x8 q8reg[QK8 ? D / 64 : 1];
    if (!QK8) {
        const uint16_t* qrow = p.q + ((qtok0 + ti) * p.Hq + hh) * D;
#pragma unroll
        for (int dc = 0; dc < D / 16; ++dc) {
            u32x4 w = *(const u32x4*)(qrow + dc * 16 + half * 8);
            w = (w & p.qand) ^ p.qsign;
            qreg[dc] = __builtin_bit_cast(bf16x8, w);
        }
    } else {
        const uint8_t* qrow = (const uint8_t*)p.q + ((qtok0 + ti) * p.Hq + hh) * D;
#pragma unroll
        for (int t = 0; t < D / 64; ++t) {
            const u32x4 w0 = (*(const u32x4*)(qrow + 64 * t + 32 * half) & p.qand) ^ p.qsign;
            const u32x4 w1 = (*(const u32x4*)(qrow + 64 * t + 32 * half + 16) & p.qand) ^ p.qsign;
            q8reg[t] = i32x8{(int)w0[0], (int)w0[1], (int)w0[2], (int)w0[3], (int)w1[0], (int)w1[1], (int)w1[2], (int)w1[3]};
        }
    }

    // ---- key tile range of this work item
    const int r_last = min(r0 + kBlockM, R) - 1;
    const int i_max = (int)fdiv((uint32_t)r_last, p.gmul, p.gshift);
    int kv_end = Sk;
    if (CAUSAL) kv_end = min(Sk, i_max + koff + 1);
    const int T = kv_end > 0 ? (kv_end + kBlockN - 1) / kBlockN : 0;
    int t_begin = 0, t_end = T;
    if (SPLIT) {
        t_begin = (int)(((int64_t)s * T) / p.ns);
        t_end = (int)(((int64_t)(s + 1) * T) / p.ns);
    }

    // rows of this wave: tokens [iw_min, iw_max]
    const int rw0 = r0 + wave * 32;
    const bool wave_active = rw0 < R;
    const int iw_min = (int)fdiv((uint32_t)min(rw0, R - 1), p.gmul, p.gshift);
    const int iw_max = (int)fdiv((uint32_t)(min(rw0 + 32, R) - 1), p.gmul, p.gshift);

    // ---- K/V tile loads: per-lane byte offsets inside a tile, scalar tile base
    const int64_t kv_stride_b = (int64_t)p.Hk * D * 2;
    const int64_t k_stride_b = QK8 ? (int64_t)p.Hk * D : kv_stride_b;
    // contiguous: this sequence's rows of head g; paged: head g of pool page 0
    const char* kbase = QK8 ? (const char*)p.k + (ktok0 * p.Hk + g) * D
                            : (const char*)(p.k + (PAGED ? (int64_t)g * D : (ktok0 * p.Hk + g) * D));
    const char* vbase = (const char*)(p.v + (PAGED ? (int64_t)g * D : (ktok0 * p.Hk + g) * D));
    // chunk ci of a tile: row ci / (chunks per row), stored at its position
    // in the row, holding the global chunk that the row's swizzle puts there
    auto k_chunk = [&](int ci, int& row) {
        row = ci / (QK8 ? NCH8 : NCH);
        return QK8 ? (ci % NCH8) ^ swz8<D>(row) : (ci % NCH) ^ swz<D>(row);
    };
    uint32_t goff[NLOAD], goffk[NLOADK];
#pragma unroll
    for (int u = 0; u < NLOAD; ++u) {
        const int ci = (u * 4 + wave) * 64 + lane;
        const int row = ci / NCH;
        const int logical_ch = (ci % NCH) ^ swz<D>(row);
        goff[u] = (uint32_t)(row * kv_stride_b + logical_ch * 16);
    }
#pragma unroll
    for (int u = 0; u < NLOADK; ++u) {
        int row;
        const int logical_ch = k_chunk((u * 4 + wave) * 64 + lane, row);
        goffk[u] = (uint32_t)(row * k_stride_b + logical_ch * 16);
    }
    auto issue = [&](int kv0, int buf) {
        LDS char* kt = lds + buf * 2 * TILE_B;
        LDS char* vt = kt + TILE_B;
        if (PAGED) {
            // copy u covers key rows 64*(4u + wave)/NCH .. +64/NCH-1 of the tile
            // (4 at d=128, 8 at d=64), inside one group of 16 keys and so inside
            // one page: the page of its first row (or of the last key, past the
            // end, where every row re-reads the last key). A scalar load (constant
            // address space), so that it never waits for the copies in flight.
            const __attribute__((address_space(4))) int* table =
                (const __attribute__((address_space(4))) int*)p.block_table;
#pragma unroll
            for (int u = 0; u < NLOAD; ++u) {
                const int key_first = min(kv0 + (u * 4 + wave) * 64 / NCH, Sk - 1);
                const int pidx = (int)fdiv((uint32_t)key_first, p.pmul, p.pshift);
                const int page = __builtin_amdgcn_readfirstlane(
                    min(max(table[(int64_t)b * p.max_pages + pidx], 0), p.num_pages - 1));
                const int64_t page_off = (int64_t)page * p.page_size * kv_stride_b;
                uint32_t off;
                if (kv0 + kBlockN <= Sk) {  // full tile: the copy's rows start at or after the page's first key
                    off = goff[u] - (uint32_t)((pidx * p.page_size - kv0) * kv_stride_b);
                } else {
                    const int ci = (u * 4 + wave) * 64 + lane;
                    const int row = ci / NCH;
                    const int logical_ch = (ci % NCH) ^ swz<D>(row);
                    const int key = min(kv0 + row, Sk - 1) - pidx * p.page_size;
                    off = (uint32_t)(key * kv_stride_b + logical_ch * 16);
                }
                lds_dma16(kbase + page_off, off, kt + (u * 4 + wave) * 1024);
                lds_dma16(vbase + page_off, off, vt + (u * 4 + wave) * 1024);
            }
            return;
        }
        const char* kg = kbase + kv0 * k_stride_b;
        const char* vg = vbase + kv0 * kv_stride_b;
        // copy u of K (fp8: the first NLOADK) and of V go to the same offset of
        // their tiles; with bf16 K the two copies of each u are issued together
        if (kv0 + kBlockN <= Sk) {
#pragma unroll
            for (int u = 0; u < NLOAD; ++u) {
                if (u < NLOADK) lds_dma16(kg, goffk[u < NLOADK ? u : 0], kt + (u * 4 + wave) * 1024);
                lds_dma16(vg, goff[u], vt + (u * 4 + wave) * 1024);
            }
        } else {  // ragged last tile: rows past the end re-read the last key (masked later)
#pragma unroll
            for (int u = 0; u < NLOAD; ++u) {
                if (u < NLOADK) {
                    int row;
                    const int logical_ch = k_chunk((u * 4 + wave) * 64 + lane, row);
                    const int key = min(kv0 + row, Sk - 1) - kv0;
                    lds_dma16(kg, (uint32_t)(key * k_stride_b + logical_ch * 16), kt + (u * 4 + wave) * 1024);
                }
                const int ci = (u * 4 + wave) * 64 + lane;
                const int row = ci / NCH;
                const int logical_ch = (ci % NCH) ^ swz<D>(row);
                const int key = min(kv0 + row, Sk - 1) - kv0;
                lds_dma16(vg, (uint32_t)(key * kv_stride_b + logical_ch * 16), vt + (u * 4 + wave) * 1024);
            }
        }
    };

    // ---- per-lane LDS operand offsets (bytes, relative to the tile start)
    const int krow0 = pi32(col);
    uint32_t kofs[QK8 ? 1 : D / 16];
    uint32_t kofs8[QK8 ? D / 64 : 1][2];  // fp8: operand t, 16-byte halves of the lane's 32 bytes
    if (!QK8) {
#pragma unroll
        for (int dc = 0; dc < D / 16; ++dc) kofs[dc] = krow0 * (D * 2) + (((2 * dc + half) ^ swz<D>(krow0)) * 16);
    } else {
#pragma unroll
        for (int t = 0; t < D / 64; ++t)
#pragma unroll
            for (int e = 0; e < 2; ++e) kofs8[t][e] = krow0 * D + (((4 * t + 2 * half + e) ^ swz8<D>(krow0)) * 16);
    }
    const int u16 = lane & 15, qq = (lane >> 4) & 1;
    const int rho = ((u16 & 1) << 1) | ((u16 >> 1) & 1);  // 0,2,1,3
    uint32_t vofs[D / 32][2];
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
            const int vrow = half * 8 + rr * 4 + (u16 >> 2);   // + 16*kk, which keeps the swizzle
            const int vcol = cb * 32 + qq * 16 + rho * 4;
            vofs[cb][rr] = vrow * (D * 2) + (((vcol >> 3) ^ swz<D>(vrow)) * 16) + (vcol & 7) * 2;
        }

    f32x16 oacc[D / 32];
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) oacc[cb] = f32x16{};
    float m_run = -__builtin_inff();  // running max, scaled log2 units
    float l_part[4] = {0.f, 0.f, 0.f, 0.f};  // this lane's partial row sums (fp32 P: the LSE)
    float w_part[4] = {0.f, 0.f, 0.f, 0.f};  // ... of the bf16 P the output product uses (its normaliser)
    const float c = p.c;
    const int jlim = CAUSAL ? min(Sk - 1, ti + koff) : Sk - 1;  // last key visible to this row

    // One key tile: scores, online softmax, output update. `buf` selects the
    // LDS stage; `need_mask` is uniform across the wave.
    auto compute = [&](int buf, int kv0, bool need_mask) {
        const LDS char* kt = lds + buf * 2 * TILE_B;
        const LDS char* vt = kt + TILE_B;

        // S^T = K Q^T: two blocks of 32 keys (masked where needed)
        f32x16 sacc[2];
        auto scores = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            sacc[mb] = f32x16{};
            if (!QK8) {
#pragma unroll
                for (int dc = 0; dc < D / 16; ++dc) {
                    const bf16x8 a = *(const LDS bf16x8*)(kt + kofs[dc] + mb * 32 * D * 2);
                    sacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[dc], sacc[mb], 0, 0, 0);
                }
            } else {
#pragma unroll
                for (int t = 0; t < D / 64; ++t) {
                    const u32x4 a0 = *(const LDS u32x4*)(kt + kofs8[t][0] + mb * 32 * D);
                    const u32x4 a1 = *(const LDS u32x4*)(kt + kofs8[t][1] + mb * 32 * D);
                    const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
                    // e4m3 x e4m3 (format 0 for A and B), block scale exponents 127 = 1.0
                    sacc[mb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, q8reg[t], sacc[mb], 0, 0, 0, 127, 0, 127);
                }
            }
        }
        // keys of this lane's slots: kv0 + 32*mb + 16*(i/8) + 8*half + (i%8)
        if (need_mask) {
            const int lim = jlim - kv0 - half * 8;
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (mb * 32 + ((i >> 3) << 4) + (i & 7) > lim) sacc[mb][i] = -__builtin_inff();
        }
        };
        scores();
        // online softmax: the running maximum is raised only for rows that
        // need it (softmax_exps, always on a row's first visible key); then
        // the wavefront forms the scores again from the tile still in LDS
        // (bf16 at d=128 also on the item's first tile: keeping the first
        // scores live past the fast path spilled registers there)
        bf16x8 pk[4];
        float tl[4];
        if constexpr (D == 64 || QK8) {
            // registers to spare: a wavefront whose rows have all seen no
            // key yet (the item's first tile) finds the maximum directly
            bool need = true, redo = true;
            if (__ballot(m_run == -__builtin_inff()) != __builtin_amdgcn_read_exec()) {
                need = softmax_exps(sacc, c, m_run, tl, pk);
                redo = __ballot(need) != 0;
                if (redo) scores();
            }
            if (redo) softmax_raise(sacc, c, m_run, need, l_part, w_part, oacc, tl, pk);
        } else {
            const bool need = softmax_exps(sacc, c, m_run, tl, pk);
            if (__ballot(need)) {
                scores();
                softmax_raise(sacc, c, m_run, need, l_part, w_part, oacc, tl, pk);
            }
        }
        softmax_commit(l_part, w_part, tl, pk);

        // O^T += V^T P^T
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
            for (int cb = 0; cb < D / 32; ++cb) {
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS s16x4*)(vt + vofs[cb][0] + kk * 16 * D * 2));
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS s16x4*)(vt + vofs[cb][1] + kk * 16 * D * 2));
                const s16x8 av = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), pk[kk],
                                                                     oacc[cb], 0, 0, 0);
            }
        }
    };

    // both stages are free at the start: the first two tiles are copied
    // together (for short items the second tile's latency is not exposed)
    if (t_begin < t_end) issue(t_begin * kBlockN, 0);
    if (t_begin + 1 < t_end) issue((t_begin + 1) * kBlockN, 1);
    for (int t = t_begin; t < t_end; ++t) {
        const int buf = (t - t_begin) & 1;
        wait_vmem();
        __syncthreads();
        if (t > t_begin && t + 1 < t_end) issue((t + 1) * kBlockN, buf ^ 1);
        const int kv0 = t * kBlockN;
        // waves whose rows see none of these keys skip the arithmetic
        if (wave_active && !(CAUSAL && kv0 > iw_max + koff)) {
            const bool need_mask = (kv0 + kBlockN > Sk) || (CAUSAL && kv0 + kBlockN - 1 > iw_min + koff);
            compute(buf, kv0, need_mask);
        }
    }

    // ---- epilogue
    // O is normalised by the sum of the bf16 probabilities its product used;
    // the LSE comes from the fp32 probabilities. A split writes both log-sums:
    // the combine weights its outputs by the first and merges the LSE from the
    // second, which reproduces the unsplit arithmetic.
    const float l_tot = xhalf_sum((l_part[0] + l_part[1]) + (l_part[2] + l_part[3]));
    const float w_tot = xhalf_sum((w_part[0] + w_part[1]) + (w_part[2] + w_part[3]));
    const bool live = l_tot > 0.f;  // the largest probability is >= 1/2, so w_tot > 0 too
    const float inv = live ? 1.f / w_tot : 0.f;
    const float lse_val = live ? (m_run + __log2f(l_tot)) * kLn2 : -__builtin_inff();
    const int64_t grow = (qtok0 + ti) * p.Hq + hh;  // row of [B*Sq or total_q, Hq]
    if (!SPLIT) {
        if (row_valid) {
            uint16_t* orow = p.o + grow * D;
#pragma unroll
            for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
                for (int run = 0; run < 2; ++run) {
                    bf16x8 ov;
#pragma unroll
                    for (int i = 0; i < 8; ++i) ov[i] = (__bf16)(oacc[cb][run * 8 + i] * inv);
                    *(bf16x8*)(orow + cb * 32 + run * 16 + half * 8) = ov;
                }
            if (half == 0 && p.lse) p.lse[lse_index(p, b, hh, qtok0, ti, VARLEN)] = lse_val;
        }
    } else {
        if (row_valid) {
            const int64_t rows = VARLEN ? (int64_t)p.total_q * p.Hq : (int64_t)p.B * p.Sq * p.Hq;
            float* orow = p.opart + ((int64_t)s * rows + grow) * D;
#pragma unroll
            for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
                for (int run = 0; run < 2; ++run) {
                    f32x4 v0, v1;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        v0[i] = oacc[cb][run * 8 + i] * inv;
                        v1[i] = oacc[cb][run * 8 + 4 + i] * inv;
                    }
                    float* dst = orow + cb * 32 + run * 16 + half * 8;
                    *(f32x4*)dst = v0;
                    *(f32x4*)(dst + 4) = v1;
                }
            if (half == 0) {
                p.lpart[(int64_t)s * rows + grow] = lse_val;
                p.wpart[(int64_t)s * rows + grow] = live ? (m_run + __log2f(w_tot)) * kLn2 : -__builtin_inff();
            }
        }
    }
}

// Large prefill launches (unsplit bf16 calls at d=128 with enough work items
// to fill the GPU): the same per-row arithmetic as attn_fwd_kernel, bit for bit, on a
// workgroup of 8 wavefronts and 256 packed rows that owns its compute unit.
// The hardware places wavefronts w and w+4 of a workgroup on the same SIMD,
// so waves 0-3 (group A) and 4-7 (group B) pair up per SIMD. Every key tile t
// takes two phases; in each phase one group issues matrix products and the
// other group runs its softmax, then they swap:
//
//   phase 2t  : A: S(t) = K(t) Q^T, then O += V(t-1)^T P(t-1)   B: softmax(t-1)
//   phase 2t+1: A: softmax(t)                                  B: S(t), O += V(t-1)^T P(t-1)
//
// so the SIMD's matrix core always has one wavefront feeding it while the
// other one works on its exponentials. A workgroup barrier starts each tile;
// the two phases are separated by a second one only in non-causal launches
// (measured on MI355X, Llama-2 heads, S=2048: without it causal calls run
// 1.5-3.5% faster at B=4..256, non-causal B=64 0.8% slower; no wavefront
// reads what the other group writes between the two). The wavefront in its
// product phase raises its issue priority (s_setprio) so the softmax
// wavefront's VALU work does not delay its products. S(t)'s K operands are
// read from LDS eight products ahead. K/V tiles stream through a ring of
// kPPStages LDS stages by global_load_lds: the copies of tile t+2 go into the
// stage of tile t-2 (whose last readers finished before tile t's barrier),
// issued by each group during its softmax phase of tile t, and a workgroup
// waits only for tile t's copies at its top. Causal masking, the row/key bookkeeping, the lazy online
// softmax in base 2 and the epilogue are those of attn_fwd_kernel.
//
// Causal launches whose pairs still give every compute unit one (p.pair_rows)
// give a workgroup two row tiles of one (batch, head unit), rt and its
// mirror row_tiles-1-rt (variable-length calls: of one sequence, from the
// work list), so that every workgroup reads about the same number of key
// tiles; the second item's Q rows are copied into LDS during the
// first item's last two tiles and its first K/V tile while the first drains.
//
// QK8 (fp8 e4m3 Q and K, contiguous batched calls): the scores run on the
// fp8 matrix cores as in attn_fwd_kernel's QK8 instantiation (the fp8 K tile
// fills the first half of its stage slot, with that kernel's swizzle), and
// the light item of a pair loads its own Q rows.
template <int D, bool CAUSAL, bool PAGED, bool VARLEN, bool QK8>
__global__ __launch_bounds__(kPPThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_fwd_pingpong_kernel(
    const FwdParams p) {
    static_assert(!(PAGED && VARLEN), "paged calls have one query length");
    static_assert(!QK8 || (!PAGED && !VARLEN), "fp8 Q/K: contiguous batched calls");
    constexpr int TILE = kBlockN * D;
    constexpr int TILE_B = TILE * 2;
    constexpr int NCH = D / 8;
    constexpr int NLOAD = kBlockN * NCH / kPPThreads;  // 16-byte copies per thread per tensor and tile
    constexpr int NCH8 = D / 16;                       // 16-byte chunks per fp8 K row
    constexpr int NLOADK = QK8 ? kBlockN * NCH8 / kPPThreads : NLOAD;  // ... of the K tile
    constexpr int NS = kPPStages;
    constexpr int COPIES = NLOADK + NLOAD;
    static_assert(NS == 4, "the stage reuse and the wait counts below assume 4 stages");
    static_assert(kPPThreads == 512 && kPPBlockM == 256, "8 wavefronts of 32 rows");
    static_assert(D == 128, "a 256-row Q tile fills two ring stages");
    __shared__ __attribute__((aligned(16))) uint16_t smem[NS * 2 * TILE];
    LDS char* lds = (LDS char*)smem;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2;
    const int lane = tid & 63;
    const int col = lane & 31, half = lane >> 5;

    // ---- work: a pair of row tiles of one (batch, head unit), the heavy one
    // (rt1, descending) first and its light partner rt2 = row_tiles-1-rt1 after
    // it; variable-length calls: an entry of the scheduling kernel's work list
    // (causal: the pair of row tiles R_b-1-pr and pr of sequence b)
    int rt1, rt2 = -1, unit, b;
    if (!VARLEN && (!CAUSAL || !p.pair_rows)) {  // one item per workgroup, heaviest first
        const int logical = xcd_remap(blockIdx.x, p.grid);
        rt1 = p.row_tiles - 1 - (logical % p.row_tiles);
        const int tmpu = logical / p.row_tiles;
        unit = tmpu % p.units_per_b;
        b = tmpu / p.units_per_b;
    } else if (!VARLEN) {
        const int npairs = (p.row_tiles + 1) >> 1;
        const int logical = xcd_remap(blockIdx.x, p.grid);
        const int pr = logical % npairs;
        const int tmpu = logical / npairs;
        unit = tmpu % p.units_per_b;
        b = tmpu / p.units_per_b;
        rt1 = p.row_tiles - 1 - pr;
        if (pr < rt1) rt2 = pr;
    } else {
        typedef const __attribute__((address_space(4))) int* cint_p;
        const cint_p wl = (cint_p)p.worklist;
        const int pair = (int)blockIdx.x / p.units_per_b;
        unit = (int)blockIdx.x % p.units_per_b;
        if (pair >= wl[0]) return;  // uniform over the workgroup
        b = __builtin_amdgcn_readfirstlane(wl[1 + 2 * pair]);
        rt1 = __builtin_amdgcn_readfirstlane(wl[2 + 2 * pair]);  // causal: pr
    }
    const int g = p.Gp > 1 ? unit : unit / p.G;
    const int h0 = p.Gp > 1 ? unit * p.G : unit;
    int Sq = p.Sq, Sk = p.Sk;
    int64_t qtok0 = (int64_t)b * p.Sq, ktok0 = (int64_t)b * p.Sk;
    if (VARLEN) seq_extent(p, b, qtok0, Sq, ktok0, Sk);
    if (PAGED) Sk = __builtin_amdgcn_readfirstlane(min(max(p.seqlens_k[b], 0), p.max_pages * p.page_size));
    const int R = VARLEN ? Sq * p.Gp : p.R;
    const int koff = Sk - Sq;  // bottom-right causal offset
    if (VARLEN && CAUSAL) {
        const int pr = rt1;
        rt1 = (R + kPPBlockM - 1) / kPPBlockM - 1 - pr;
        if (pr < rt1) rt2 = pr;
    }

    // ---- K/V tile copies: fixed per-thread 16-byte chunks, scalar tile base
    const int64_t kv_stride_b = (int64_t)p.Hk * D * 2;
    const int64_t k_stride_b = QK8 ? (int64_t)p.Hk * D : kv_stride_b;
    const char* kbase = QK8 ? (const char*)p.k + (ktok0 * p.Hk + g) * D
                            : (const char*)(p.k + (PAGED ? (int64_t)g * D : (ktok0 * p.Hk + g) * D));
    const char* vbase = (const char*)(p.v + (PAGED ? (int64_t)g * D : (ktok0 * p.Hk + g) * D));
    uint32_t goff[NLOAD];
#pragma unroll
    for (int u = 0; u < NLOAD; ++u) {
        const int ci = (u * 8 + wave) * 64 + lane;
        const int row = ci / NCH;
        const int logical_ch = (ci % NCH) ^ swz<D>(row);
        goff[u] = (uint32_t)(row * kv_stride_b + logical_ch * 16);
    }
    // fp8 K: chunk ci of the tile is row ci / NCH8, stored at its position in
    // the row, holding the global chunk the row's swizzle puts there
    uint32_t goffk[QK8 ? NLOADK : 1];
    if constexpr (QK8) {
#pragma unroll
        for (int u = 0; u < NLOADK; ++u) {
            const int ci = (u * 8 + wave) * 64 + lane;
            const int row = ci / NCH8;
            goffk[u] = (uint32_t)(row * k_stride_b + ((ci % NCH8) ^ swz8<D>(row)) * 16);
        }
    }
    // ---- per-lane LDS operand offsets (as in attn_fwd_kernel)
    const int krow0 = pi32(col);
    uint32_t kofs[QK8 ? 1 : D / 16];
    uint32_t kofs8[QK8 ? D / 64 : 1][2];  // fp8: operand t, 16-byte halves of the lane's 32 bytes
    if constexpr (!QK8) {
#pragma unroll
        for (int dc = 0; dc < D / 16; ++dc) kofs[dc] = krow0 * (D * 2) + (((2 * dc + half) ^ swz<D>(krow0)) * 16);
    } else {
#pragma unroll
        for (int t = 0; t < D / 64; ++t)
#pragma unroll
            for (int e = 0; e < 2; ++e) kofs8[t][e] = krow0 * D + (((4 * t + 2 * half + e) ^ swz8<D>(krow0)) * 16);
    }
    const int u16 = lane & 15, qq = (lane >> 4) & 1;
    const int rho = ((u16 & 1) << 1) | ((u16 >> 1) & 1);
    uint32_t vofs[D / 32][2];
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
            const int vrow = half * 8 + rr * 4 + (u16 >> 2);
            const int vcol = cb * 32 + qq * 16 + rho * 4;
            vofs[cb][rr] = vrow * (D * 2) + (((vcol >> 3) ^ swz<D>(vrow)) * 16) + (vcol & 7) * 2;
        }
    const float c = p.c;

    // The light item's Q rows reach LDS by copy during the heavy item's last
    // two tiles, into the two ring stages those tiles leave unused (rows
    // 0-127 and 128-255 of the tile, 16-byte chunk ch of row r at slot
    // 16r + (ch ^ (r & 15)) of its stage), and its tile 0 during the heavy
    // item's drain step. Its ring starts two stages after the heavy item's.
    int ring = 0;          // stage of the item's tile 0
    bool q_staged = false; // the item's Q rows and tile 0 were copied by the previous item
    // the two items run as two inlined copies of one body (no loop back edge,
    // so nothing of the first item stays live into the second)
    auto do_item = [&](auto item_c) __attribute__((always_inline)) {
        constexpr int item = decltype(item_c)::value;
        const int rt = item == 0 ? rt1 : rt2;
        const int r0 = rt * kPPBlockM;
        // ---- this lane's row: token ti, head hh
        const int r = r0 + wave * 32 + col;
        const bool row_valid = r < R;
        const int rc = min(r, R - 1);
        const int ti = (int)fdiv((uint32_t)rc, p.gmul, p.gshift);
        const int hh = h0 + (rc - ti * p.Gp);
        // ---- key tiles of the item and of this wavefront's rows
        const int r_last = min(r0 + kPPBlockM, R) - 1;
        const int i_max = (int)fdiv((uint32_t)r_last, p.gmul, p.gshift);
        int kv_end = Sk;
        if (CAUSAL) kv_end = min(Sk, i_max + koff + 1);
        const int nt = kv_end > 0 ? (kv_end + kBlockN - 1) / kBlockN : 0;
        const int rw0 = r0 + wave * 32;
        const bool wave_active = rw0 < R;
        const int iw_min = (int)fdiv((uint32_t)min(rw0, R - 1), p.gmul, p.gshift);
        const int iw_max = (int)fdiv((uint32_t)(min(rw0 + 32, R) - 1), p.gmul, p.gshift);
        // the next item (if any) is staged through LDS when this one has at least two tiles
        const bool stage_next = !QK8 && item == 0 && rt2 >= 0 && nt >= 2;

        // tile t of the item (t may run past nt-1 only through issue_next below)
        auto issue_kv = [&](int t, int ring_of_t) __attribute__((always_inline)) {
            const int kv0 = t * kBlockN;
            // the LDS destination is uniform; it is passed through a scalar register
            auto dst = [&](int tensor, int u) __attribute__((always_inline)) {
                const uint32_t a = (uint32_t)(size_t)(lds + ((ring_of_t + t) & (NS - 1)) * 2 * TILE_B + tensor * TILE_B) + (u * 8 + wave) * 1024;
                return (LDS void*)(size_t)__builtin_amdgcn_readfirstlane(a);
            };
            if (PAGED) {
                const __attribute__((address_space(4))) int* table =
                    (const __attribute__((address_space(4))) int*)p.block_table;
#pragma unroll
                for (int u = 0; u < NLOAD; ++u) {
                    const int key_first = min(kv0 + (u * 8 + wave) * 64 / NCH, Sk - 1);
                    const int pidx = (int)fdiv((uint32_t)key_first, p.pmul, p.pshift);
                    const int page = __builtin_amdgcn_readfirstlane(
                        min(max(table[(int64_t)b * p.max_pages + pidx], 0), p.num_pages - 1));
                    const int64_t page_off = (int64_t)page * p.page_size * kv_stride_b;
                    uint32_t off;
                    if (kv0 + kBlockN <= Sk) {
                        off = goff[u] - (uint32_t)((pidx * p.page_size - kv0) * kv_stride_b);
                    } else {
                        const int ci = (u * 8 + wave) * 64 + lane;
                        const int row = ci / NCH;
                        const int logical_ch = (ci % NCH) ^ swz<D>(row);
                        const int key = min(kv0 + row, Sk - 1) - pidx * p.page_size;
                        off = (uint32_t)(key * kv_stride_b + logical_ch * 16);
                    }
                    lds_dma16(kbase + page_off, off, dst(0, u));
                    lds_dma16(vbase + page_off, off, dst(1, u));
                }
                return;
            }
            const char* kg = kbase + kv0 * k_stride_b;
            const char* vg = vbase + kv0 * kv_stride_b;
            if constexpr (QK8) {
                if (kv0 + kBlockN <= Sk) {
#pragma unroll
                    for (int u = 0; u < NLOADK; ++u) lds_dma16(kg, goffk[u], dst(0, u));
#pragma unroll
                    for (int u = 0; u < NLOAD; ++u) lds_dma16(vg, goff[u], dst(1, u));
                } else {  // ragged last tile: rows past the end re-read the last key (masked later)
#pragma unroll
                    for (int u = 0; u < NLOADK; ++u) {
                        const int ci = (u * 8 + wave) * 64 + lane;
                        const int row = ci / NCH8;
                        const int key = min(kv0 + row, Sk - 1) - kv0;
                        lds_dma16(kg, (uint32_t)(key * k_stride_b + ((ci % NCH8) ^ swz8<D>(row)) * 16), dst(0, u));
                    }
#pragma unroll
                    for (int u = 0; u < NLOAD; ++u) {
                        const int ci = (u * 8 + wave) * 64 + lane;
                        const int row = ci / NCH;
                        const int key = min(kv0 + row, Sk - 1) - kv0;
                        lds_dma16(vg, (uint32_t)(key * kv_stride_b + ((ci % NCH) ^ swz<D>(row)) * 16), dst(1, u));
                    }
                }
                return;
            }
            if (kv0 + kBlockN <= Sk) {
#pragma unroll
                for (int u = 0; u < NLOAD; ++u) {
                    lds_dma16(kg, goff[u], dst(0, u));
                    lds_dma16(vg, goff[u], dst(1, u));
                }
            } else {
#pragma unroll
                for (int u = 0; u < NLOAD; ++u) {
                    const int ci = (u * 8 + wave) * 64 + lane;
                    const int row = ci / NCH;
                    const int logical_ch = (ci % NCH) ^ swz<D>(row);
                    const int key = min(kv0 + row, Sk - 1) - kv0;
                    const uint32_t off = (uint32_t)(key * kv_stride_b + logical_ch * 16);
                    lds_dma16(kg, off, dst(0, u));
                    lds_dma16(vg, off, dst(1, u));
                }
            }
        };
        auto issue = [&](int t) __attribute__((always_inline)) { issue_kv(t, ring); };
        // half `part` (rows 128*part ..) of the next item's Q tile into stage ring+nt+part
        auto issue_next_q = [&](int part) __attribute__((always_inline)) {
            const uint32_t sbase = (uint32_t)(size_t)(lds + ((ring + nt + part) & (NS - 1)) * 2 * TILE_B);
            // offsets from the item's first token: at most 256 tokens of Hq rows
            const int tok_first = (int)fdiv((uint32_t)min(rt2 * kPPBlockM, R - 1), p.gmul, p.gshift);
            const char* qb = (const char*)(p.q + (qtok0 + tok_first) * p.Hq * D);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int slot = (u * 8 + wave) * 64 + lane;  // 16-byte slot of the stage
                const int rl = slot >> 4;                      // row of the half
                const int ch = (slot & 15) ^ (rl & 15);
                const int rq = min(rt2 * kPPBlockM + part * 128 + rl, R - 1);
                const int tq = (int)fdiv((uint32_t)rq, p.gmul, p.gshift);
                const int hq = h0 + (rq - tq * p.Gp);
                const uint32_t off = (uint32_t)((((tq - tok_first) * p.Hq + hq) * D * 2) + ch * 16);
                lds_dma16(qb, off, (LDS void*)(size_t)__builtin_amdgcn_readfirstlane(sbase + (u * 8 + wave) * 1024));
            }
        };

        // ---- prologue: the Q rows (B operand of S^T = K Q^T), tiles 0 and 1
        bf16x8 qreg[QK8 ? 1 : D / 16];
        i32x8 q8reg[QK8 ? D / 64 : 1];  // fp8: operand t holds d 64t .. 64t+63, lane half h bytes 32h ..
        if constexpr (QK8) {
            if (item > 0) __syncthreads();  // every wavefront is done with the previous item's stages
            if (nt > 0) issue(0);
            const uint8_t* qrow = (const uint8_t*)p.q + ((qtok0 + ti) * p.Hq + hh) * D;
#pragma unroll
            for (int t = 0; t < D / 64; ++t) {
                const u32x4 w0 = (*(const u32x4*)(qrow + 64 * t + 32 * half) & p.qand) ^ p.qsign;
                const u32x4 w1 = (*(const u32x4*)(qrow + 64 * t + 32 * half + 16) & p.qand) ^ p.qsign;
                // wait for Q here (16-byte operands: the host pass checks the constraint too)
                asm volatile("" ::"v"(w0), "v"(w1));
                q8reg[t] = i32x8{(int)w0[0], (int)w0[1], (int)w0[2], (int)w0[3], (int)w1[0], (int)w1[1], (int)w1[2], (int)w1[3]};
            }
            if (nt > 1) issue(1);
        } else if (!q_staged) {
            if (item > 0) __syncthreads();  // every wavefront is done with the previous item's stages
            if (nt > 0) issue(0);
            const uint16_t* qrow = p.q + ((qtok0 + ti) * p.Hq + hh) * D;
#pragma unroll
            for (int dc = 0; dc < D / 16; ++dc) {
                u32x4 w = *(const u32x4*)(qrow + dc * 16 + half * 8);
                w = (w & p.qand) ^ p.qsign;
                qreg[dc] = __builtin_bit_cast(bf16x8, w);
            }
            // wait for Q here, before the tile loop, so that no wait on it lands inside
#pragma unroll
            for (int dc = 0; dc < D / 16; ++dc) asm volatile("" ::"v"(qreg[dc]));
            if (nt > 1) issue(1);
        } else {
            // this thread's Q copies landed before the previous item's stores;
            // the barrier makes every thread's copies visible and frees the
            // previous item's last stage
            __syncthreads();
            const int rl = wave * 32 + col, part = rl >> 7, rh = rl & 127;
            const LDS char* qs = lds + ((ring - 2 + part) & (NS - 1)) * 2 * TILE_B + rh * 256;
#pragma unroll
            for (int dc = 0; dc < D / 16; ++dc) {
                u32x4 w = *(const LDS u32x4*)(qs + (((2 * dc + half) ^ (rh & 15)) * 16));
                w = (w & p.qand) ^ p.qsign;
                qreg[dc] = __builtin_bit_cast(bf16x8, w);
            }
#pragma unroll
            for (int dc = 0; dc < D / 16; ++dc) asm volatile("" ::"v"(qreg[dc]));
            wait_vmem();  // tile 0 (and the previous item's stores)
            if (nt > 1) issue(1);
        }

        f32x16 oacc[D / 32];
#pragma unroll
        for (int cb = 0; cb < D / 32; ++cb) oacc[cb] = f32x16{};
        float m_run = -__builtin_inff();  // running max, scaled log2 units
        float l_part[4] = {0.f, 0.f, 0.f, 0.f};  // fp32 P: the LSE
        float w_part[4] = {0.f, 0.f, 0.f, 0.f};  // bf16 P: the output's normaliser
        const int jlim = CAUSAL ? min(Sk - 1, ti + koff) : Sk - 1;  // last key visible to this row
        f32x16 sacc[2];
        bf16x8 pk[4];
        // waves whose rows see none of tile t's keys skip its arithmetic (monotone in t)
        auto act = [&](int t) __attribute__((always_inline)) {
            return wave_active && !(CAUSAL && t * kBlockN > iw_max + koff);
        };
        auto s_part = [&](int t) __attribute__((always_inline)) {
            const LDS char* kt = lds + ((ring + t) & (NS - 1)) * 2 * TILE_B;
    #pragma unroll
            for (int mb = 0; mb < 2; ++mb) sacc[mb] = f32x16{};
            if constexpr (QK8) {  // all eight operand reads first, then the four fp8 products
                i32x8 a[2][D / 64];
    #pragma unroll
                for (int mb = 0; mb < 2; ++mb)
    #pragma unroll
                    for (int tt = 0; tt < D / 64; ++tt) {
                        const u32x4 a0 = *(const LDS u32x4*)(kt + kofs8[tt][0] + mb * 32 * D);
                        const u32x4 a1 = *(const LDS u32x4*)(kt + kofs8[tt][1] + mb * 32 * D);
                        a[mb][tt] = i32x8{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
                    }
    #pragma unroll
                for (int mb = 0; mb < 2; ++mb)
    #pragma unroll
                    for (int tt = 0; tt < D / 64; ++tt)
                        // e4m3 x e4m3 (format 0 for A and B), block scale exponents 127 = 1.0
                        sacc[mb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[mb][tt], q8reg[tt], sacc[mb], 0, 0, 0, 127, 0, 127);
                return;
            }
    #pragma unroll
            for (int dc = 0; dc < D / 16; ++dc)
    #pragma unroll
                for (int mb = 0; mb < 2; ++mb) {
                    const bf16x8 a = *(const LDS bf16x8*)(kt + kofs[dc] + mb * 32 * D * 2);
                    sacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[dc], sacc[mb], 0, 0, 0);
                }
            // the operand reads run eight ahead of the products
            constexpr int NR = D / 8, PRE = 8;
            __builtin_amdgcn_sched_group_barrier(0x100, PRE, 0);
    #pragma unroll
            for (int i = 0; i < (NR - PRE) / 2; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, PRE, 0);
        };
        auto pv_part = [&](int t) __attribute__((always_inline)) {
            const LDS char* vt = lds + ((ring + t) & (NS - 1)) * 2 * TILE_B + TILE_B;
    #pragma unroll
            for (int kk = 0; kk < 4; ++kk)
    #pragma unroll
                for (int cb = 0; cb < D / 32; ++cb) {
                    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS s16x4*)(vt + vofs[cb][0] + kk * 16 * D * 2));
                    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS s16x4*)(vt + vofs[cb][1] + kk * 16 * D * 2));
                    const s16x8 av = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                    oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), pk[kk], oacc[cb], 0, 0, 0);
                }
        };
        auto mask = [&](int t) __attribute__((always_inline)) {
            const int kv0 = t * kBlockN;
            const bool need_mask = (kv0 + kBlockN > Sk) || (CAUSAL && kv0 + kBlockN - 1 > iw_min + koff);
            // keys of this lane's slots: kv0 + 32*mb + 16*(i/8) + 8*half + (i%8)
            if (need_mask) {
                const int lim = jlim - kv0 - half * 8;
    #pragma unroll
                for (int mb = 0; mb < 2; ++mb)
    #pragma unroll
                    for (int i = 0; i < 16; ++i)
                        if (mb * 32 + ((i >> 3) << 4) + (i & 7) > lim) sacc[mb][i] = -__builtin_inff();
            }
        };
        // the online softmax of attn_fwd_kernel, row for row (O holds every
        // product up to tile t-1 here). A wavefront whose rows have all seen
        // no key yet finds the row maximum directly; otherwise, when a row
        // needs a raise of its maximum, the scores are formed again from tile
        // t, still in LDS. Either way each row takes the same steps as there.
        auto softmax = [&](int t) __attribute__((always_inline)) {
            mask(t);
            float tl[4];
            bool need = true, redo = true;
            if (__ballot(m_run == -__builtin_inff()) != __builtin_amdgcn_read_exec()) {
                need = softmax_exps(sacc, c, m_run, tl, pk);
                redo = __ballot(need) != 0;
                if (redo) {
                    s_part(t);
                    mask(t);
                }
            }
            if (redo) softmax_raise(sacc, c, m_run, need, l_part, w_part, oacc, tl, pk);
            softmax_commit(l_part, w_part, tl, pk);
        };
        auto product_phase = [&](int t) __attribute__((always_inline)) {
            __builtin_amdgcn_s_setprio(1);
            if (t < nt && act(t)) s_part(t);
            if (t > 0 && act(t - 1)) pv_part(t - 1);
            __builtin_amdgcn_s_setprio(0);
        };
        // softmax phase of tile t (any t in [-1, nt]); the copies of tile t+2 go first
        auto softmax_phase = [&](int t_copy, int t_soft) __attribute__((always_inline)) {
            if (t_copy + NS - 2 < nt) issue(t_copy + NS - 2);
            else if (stage_next && t_copy + NS - 2 < nt + 2) issue_next_q(t_copy + NS - 2 - nt);
            else if (stage_next && t_copy + NS - 2 == nt + 2) {
                // the Q copies of this thread land first, then the next item's tile 0 goes out
                wait_vmem();
                issue_kv(0, ring + nt + 2);
            }
            if (t_soft >= 0 && t_soft < nt && act(t_soft)) softmax(t_soft);
        };
        // top of tile t: this thread's copies of tile t have landed (at most tile
        // t+1's copies are still in flight), then the barrier publishes the tile
        // and frees the stage of tile t-2
        auto top = [&](int t) __attribute__((always_inline)) {
            if (t < nt) {
                if (t + 1 < nt) wait_vmem_n<COPIES>();
                else wait_vmem();
            }
            __syncthreads();
        };
        // the two groups run separate copies of the loop, so the compiler never
        // merges two versions of the accumulators at a branch join
        auto run = [&](auto is_b) __attribute__((always_inline)) {
            for (int t = 0; t <= nt; ++t) {
                top(t);
                if (!decltype(is_b)::value) product_phase(t);
                else softmax_phase(t, t - 1);
                if (!CAUSAL) __syncthreads();
                if (!decltype(is_b)::value) softmax_phase(t, t);
                else product_phase(t);
            }
        };
        if (grp == 0) run(std::false_type{});
        else run(std::true_type{});

        // ---- epilogue
        const float l_tot = xhalf_sum((l_part[0] + l_part[1]) + (l_part[2] + l_part[3]));
        const float w_tot = xhalf_sum((w_part[0] + w_part[1]) + (w_part[2] + w_part[3]));
        const bool live = l_tot > 0.f;
        const float inv = live ? 1.f / w_tot : 0.f;
        const float lse_val = live ? (m_run + __log2f(l_tot)) * kLn2 : -__builtin_inff();
        if (row_valid) {
            uint16_t* orow = p.o + ((qtok0 + ti) * p.Hq + hh) * D;
    #pragma unroll
            for (int cb = 0; cb < D / 32; ++cb)
    #pragma unroll
                for (int run2 = 0; run2 < 2; ++run2) {
                    bf16x8 ov;
    #pragma unroll
                    for (int i = 0; i < 8; ++i) ov[i] = (__bf16)(oacc[cb][run2 * 8 + i] * inv);
                    *(bf16x8*)(orow + cb * 32 + run2 * 16 + half * 8) = ov;
                }
            if (half == 0 && p.lse) p.lse[lse_index(p, b, hh, qtok0, ti, VARLEN)] = lse_val;
        }
        ring += nt + 2;
        q_staged = stage_next;
    };
    do_item(std::integral_constant<int, 0>{});
    if (CAUSAL && rt2 >= 0) do_item(std::integral_constant<int, 1>{});
}

// Decode-shaped work (the pages' decode regime: one or a few new tokens per
// sequence against a long KV cache, bound by reading K and V from HBM): a
// head unit has at most 32 query rows (with PackGQA, the G query heads of a
// KV group times the new tokens), so one wavefront holds them all. Each
// workgroup is that single wavefront: it streams its split of the keys in
// tiles of 32 through a ring of STAGES LDS stages, keeping STAGES-1 tiles in
// flight and waiting only for the oldest (no workgroup barrier), so several
// independent workgroups per compute unit keep HBM busy. The arithmetic per
// tile is the same as in the tiled kernel (transposed MFMA products, lazy
// online softmax in base 2), on one block of 32 keys.
//
// PAGED: the keys of sequence b live in a pool of fixed-size pages (the
// pages' paged KV cache for dynamic-length sequences, Stable-Diffusion GQA
// guide, application scenario one): key j is row j % page_size of pool page
// block_table[b][j / page_size], and sequence b has seqlens_k[b] keys
// (causal alignment per sequence). page_size is a multiple of 16, so every
// 16-key half of a tile lies in one page and each copy instruction (4 or 8
// key rows) reads from one page. Lengths are clamped to the table's capacity
// and page numbers to the pool, so no input makes a read leave the buffers.
//
// KV8: K and V are stored as fp8 e4m3 (the pages' FP8 e4m3 to halve the
// bandwidth pressure, rise-and-fall tuning article, "verification and
// further directions") with per-tensor factors: the scores use
// scale * k_scale, the output is multiplied by v_scale. The ring holds the
// raw fp8 tiles (half the bytes per key). Each matrix operand is read from
// them and converted in registers: for K, 8 consecutive bytes of one key;
// for V, 8 keys of one column through the transposing byte read. Every e4m3
// value is exact in bf16 and the operands hold the same values in the same
// order (the accumulator rows of V's columns aside, which only change where
// the epilogue stores them), so the products are those of bf16 K/V holding
// the fp8 values.
template <int D, bool CAUSAL, bool SPLIT, bool PAGED, bool KV8, bool VARLEN, int STAGES>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void attn_decode_kernel(const FwdParams p) {
    constexpr int BN = kDecBlockN;                 // keys per tile
    constexpr int EB = KV8 ? 1 : 2;                // bytes per stored K/V element
    constexpr int TILE_B = BN * D * EB;            // ring bytes of one K or V tile
    constexpr int NCH = D * EB / 16;               // 16-byte chunks per stored row
    constexpr int NLOAD = BN * NCH / 64;           // 16-byte copies per lane per tensor and tile
    constexpr int RING_B = STAGES * 2 * TILE_B;
    static_assert(BN == 32, "one 32-key MFMA block per tile");
    __shared__ u32x4 smem[RING_B / 16];
    LDS char* lds = (LDS char*)smem;               // ring stage s: K tile, then V tile

    const int lane = threadIdx.x;
    const int col = lane & 31, half = lane >> 5;

    // ---- work item: (batch, head unit, split), split fastest
    const int item = blockIdx.x;
    const int s = item % p.ns;
    const int tmp = item / p.ns;
    const int unit = tmp % p.units_per_b;
    const int b = tmp / p.units_per_b;
    const int g = p.Gp > 1 ? unit : unit / p.G;   // KV head
    const int h0 = p.Gp > 1 ? unit * p.G : unit;  // first query head of the unit

    // ---- this sequence: query tokens qtok0 .. qtok0+Sq-1, keys ktok0 .. ktok0+Sk-1
    int Sq = p.Sq, Sk = p.Sk;
    int64_t qtok0 = (int64_t)b * p.Sq, ktok0 = (int64_t)b * p.Sk;
    if (VARLEN) seq_extent(p, b, qtok0, Sq, ktok0, Sk);
    if (PAGED) Sk = __builtin_amdgcn_readfirstlane(min(max(p.seqlens_k[b], 0), p.max_pages * p.page_size));
    const int R = VARLEN ? Sq * p.Gp : p.R;  // rows of this head unit
    if (VARLEN && R == 0) return;             // a sequence without queries

    // ---- this lane's row (all R <= 32 rows of the head unit): token ti, head hh
    const int r = col;
    const bool row_valid = r < R;
    const int rc = min(r, R - 1);
    const int ti = (int)fdiv((uint32_t)rc, p.gmul, p.gshift);
    const int hh = h0 + (rc - ti * p.Gp);
    const int koff = Sk - Sq;  // bottom-right causal offset

    bf16x8 qreg[D / 16];
    {
        const uint16_t* qrow = p.q + ((qtok0 + ti) * p.Hq + hh) * D;
#pragma unroll
        for (int dc = 0; dc < D / 16; ++dc) {
            u32x4 w = *(const u32x4*)(qrow + dc * 16 + half * 8);
            w = (w & p.qand) ^ p.qsign;
            qreg[dc] = __builtin_bit_cast(bf16x8, w);
        }
    }

    // ---- key tiles of this split. The unit's rows are tokens 0 .. Sq-1.
    int kv_end = Sk;
    if (CAUSAL) kv_end = min(Sk, Sq - 1 + koff + 1);
    const int T = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;
    int t_begin = 0, t_end = T;
    if (SPLIT) {
        t_begin = (int)(((int64_t)s * T) / p.ns);
        t_end = (int)(((int64_t)(s + 1) * T) / p.ns);
    }
    const int n = t_end - t_begin;

    // ---- tile copies: per-lane byte offsets inside a tile. Tiles are stored
    // swizzled: 16-byte chunk c of row r at c ^ swz(r) (bf16) or c ^ swz8(r)
    // (fp8; the 256-byte bank window holds 256/D rows of D bytes, and rows of
    // one window pair with distinct chunk masks, so 16 consecutive keys
    // reading the same logical chunk hit 16 distinct 16-byte bank slots).
    const int64_t kv_stride_b = (int64_t)p.Hk * D * EB;
    // contiguous: this sequence's rows of head g; paged: head g of page 0
    const int64_t seq_off = PAGED ? (int64_t)g * D : (ktok0 * p.Hk + g) * D;
    const char* kbase = (const char*)p.k + seq_off * EB;
    const char* vbase = (const char*)p.v + seq_off * EB;
    auto swz8 = [](int row) { return (row / (256 / D)) % (D / 16); };
    auto ring_chunk = [&](int ci, int row) { return KV8 ? ((ci % NCH) ^ swz8(row)) : ((ci % NCH) ^ swz<D>(row)); };
    uint32_t goff[NLOAD];
#pragma unroll
    for (int u = 0; u < NLOAD; ++u) {
        const int ci = u * 64 + lane;
        const int row = ci / NCH;
        goff[u] = (uint32_t)(row * kv_stride_b + ring_chunk(ci, row) * 16);
    }
    auto issue = [&](int t, int stage) {
        const int kv0 = t * BN;
        LDS char* kt = lds + stage * 2 * TILE_B;
        LDS char* vt = kt + TILE_B;
        if (PAGED) {
            // each 16-key half: the page of its first key (or of the last key
            // when the half lies past the end), rows clamped to the last key
            constexpr int RPI = 64 / NCH;  // key rows per copy instruction
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int key_first = min(kv0 + 16 * hf, Sk - 1);
                const int pidx = (int)fdiv((uint32_t)key_first, p.pmul, p.pshift);
                // scalar load (constant address space): a vector load would make
                // the compiler wait for every tile copy in flight before using it
                const __attribute__((address_space(4))) int* table =
                    (const __attribute__((address_space(4))) int*)p.block_table;
                const int page = __builtin_amdgcn_readfirstlane(
                    min(max(table[(int64_t)b * p.max_pages + pidx], 0), p.num_pages - 1));
                const int pstart = pidx * p.page_size;
                const int64_t page_off = (int64_t)page * p.page_size * kv_stride_b;
                const char* kg = kbase + page_off;
                const char* vg = vbase + page_off;
#pragma unroll
                for (int u = hf * (16 / RPI); u < (hf + 1) * (16 / RPI); ++u) {
                    const int ci = u * 64 + lane;
                    const int row = ci / NCH;
                    const int key = min(kv0 + row, Sk - 1) - pstart;
                    const uint32_t o = (uint32_t)(key * kv_stride_b + ring_chunk(ci, row) * 16);
                    lds_dma16(kg, o, kt + u * 1024);
                    lds_dma16(vg, o, vt + u * 1024);
                }
            }
            return;
        }
        const char* kg = kbase + kv0 * kv_stride_b;
        const char* vg = vbase + kv0 * kv_stride_b;
        if (kv0 + BN <= Sk) {
#pragma unroll
            for (int u = 0; u < NLOAD; ++u) {
                lds_dma16(kg, goff[u], kt + u * 1024);
                lds_dma16(vg, goff[u], vt + u * 1024);
            }
        } else {  // ragged last tile: rows past the end re-read the last key (masked later)
#pragma unroll
            for (int u = 0; u < NLOAD; ++u) {
                const int ci = u * 64 + lane;
                const int row = ci / NCH;
                const int key = min(kv0 + row, Sk - 1) - kv0;
                const uint32_t o = (uint32_t)(key * kv_stride_b + ring_chunk(ci, row) * 16);
                lds_dma16(kg, o, kt + u * 1024);
                lds_dma16(vg, o, vt + u * 1024);
            }
        }
    };

    // ---- per-lane LDS operand offsets (as in the tiled kernel, one key block;
    // fp8 K: the 8 bytes of values 16*dc + 8*half .. +7 of key krow0)
    const int krow0 = pi32(col);
    uint32_t kofs[D / 16];
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc)
        kofs[dc] = KV8 ? krow0 * D + ((dc ^ swz8(krow0)) * 16) + half * 8
                       : krow0 * (D * 2) + (((2 * dc + half) ^ swz<D>(krow0)) * 16);
    const int u16 = lane & 15, qq = (lane >> 4) & 1;
    const int rho = ((u16 & 1) << 1) | ((u16 >> 1) & 1);
    uint32_t vofs[D / 32][2];
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
            const int vrow = half * 8 + rr * 4 + (u16 >> 2);
            const int vcol = cb * 32 + qq * 16 + rho * 4;
            vofs[cb][rr] = vrow * (D * 2) + (((vcol >> 3) ^ swz<D>(vrow)) * 16) + (vcol & 7) * 2;
        }
    // fp8 V: one transposing byte read per product. In each group of 16
    // lanes, lane 2k+b names 8 bytes of key row k (of the group's 8 keys)
    // starting at column 16*(group % 2) + 8*b of the 32-column block; lane j
    // (j < 8) of the group receives byte j of the rows named by the even
    // lanes, lane 8+j byte j of the rows named by the odd lanes, i.e. the 8
    // keys of one column in key order: the A operand of the output product.
    uint32_t v8ofs[D / 32];
    {
        const int grp16 = lane >> 4, w16 = lane & 15;
        const int vkey = 8 * (grp16 >> 1) + (w16 >> 1);
#pragma unroll
        for (int cb = 0; cb < D / 32; ++cb) {
            const int dofs = cb * 32 + 16 * (grp16 & 1) + 8 * (w16 & 1);
            v8ofs[cb] = vkey * D + (((dofs >> 4) ^ swz8(vkey)) * 16) + (dofs & 15);
        }
    }

    f32x16 oacc[D / 32];
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) oacc[cb] = f32x16{};
    float m_run = -__builtin_inff();
    float l_part[4] = {0.f, 0.f, 0.f, 0.f};  // fp32 P: the LSE
    float w_part[4] = {0.f, 0.f, 0.f, 0.f};  // bf16 P: the output's normaliser
    const float c = p.c;
    const int jlim = CAUSAL ? min(Sk - 1, ti + koff) : Sk - 1;

    auto compute = [&](int stage, int kv0) {
        const LDS char* kt = lds + stage * 2 * TILE_B;
        const LDS char* vt = kt + TILE_B;
        f32x16 sacc = f32x16{};
#pragma unroll
        for (int dc = 0; dc < D / 16; ++dc) {
            bf16x8 a;
            if (KV8) {  // exact e4m3 -> bf16 of 8 values, two per conversion
                const u32x2 w = *(const LDS u32x2*)(kt + kofs[dc]);
                u32x4 cv;
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    cv[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, false));
                    cv[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, true));
                }
                a = __builtin_bit_cast(bf16x8, cv);
            } else {
                a = *(const LDS bf16x8*)(kt + kofs[dc]);
            }
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[dc], sacc, 0, 0, 0);
        }
        // slot i of this lane holds key kv0 + 16*(i/8) + 8*half + (i%8)
        if ((kv0 + BN > Sk) || (CAUSAL && kv0 + BN - 1 > koff)) {
            const int lim = jlim - kv0 - half * 8;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (((i >> 3) << 4) + (i & 7) > lim) sacc[i] = -__builtin_inff();
        }
        float t0 = fmaxf(fmaxf(sacc[0], sacc[1]), sacc[2]);
        float t1 = fmaxf(fmaxf(sacc[3], sacc[4]), sacc[5]);
        float t2 = fmaxf(fmaxf(sacc[6], sacc[7]), sacc[8]);
        float t3 = fmaxf(fmaxf(sacc[9], sacc[10]), sacc[11]);
        t0 = fmaxf(fmaxf(t0, sacc[12]), sacc[13]);
        t1 = fmaxf(fmaxf(t1, sacc[14]), sacc[15]);
        const float mx = xhalf_max(fmaxf(fmaxf(t0, t1), fmaxf(t2, t3)));
        const float mxs = (mx == -__builtin_inff()) ? -__builtin_inff() : mx * c;
        const float alpha = raise_max(m_run, mxs);
        if (__ballot(alpha != 1.f)) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                l_part[i] *= alpha;
                w_part[i] *= alpha;
            }
#pragma unroll
            for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[cb][i] *= alpha;
        }
        const float moff = (m_run == -__builtin_inff()) ? 0.f : m_run;
        bf16x8 pk[2];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float x = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[i], c, -moff));
            l_part[i & 3] += x;
            pk[i >> 3][i & 7] = (__bf16)x;
        }
        add_bf16x8(pk[0], w_part);
        add_bf16x8(pk[1], w_part);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
            for (int cb = 0; cb < D / 32; ++cb) {
                bf16x8 av;
                if (KV8) {  // keys 16*kk + .. lie 16 rows further; the row swizzle repeats every 16 rows
                    const i32x2 w = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS i32x2*)(vt + v8ofs[cb] + kk * 16 * D));
                    u32x4 cv;
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        cv[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, false));
                        cv[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, true));
                    }
                    av = __builtin_bit_cast(bf16x8, cv);
                } else {
                    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS s16x4*)(vt + vofs[cb][0] + kk * 16 * D * 2));
                    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS s16x4*)(vt + vofs[cb][1] + kk * 16 * D * 2));
                    av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                }
                oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pk[kk], oacc[cb], 0, 0, 0);
            }
        }
    };

    // ---- ring: tile j lives in stage j % STAGES. Before computing tile j the
    // wave starts tile j+STAGES-1 (into the stage tile j-1 used, whose reads
    // are complete) and waits until only the copies of the tiles after j are
    // still in flight. Copies complete in issue order.
#pragma unroll
    for (int i = 0; i < STAGES - 1; ++i)
        if (i < n) issue(t_begin + i, i);
    for (int j = 0; j < n; ++j) {
        if (j + STAGES - 1 < n) {
            issue(t_begin + j + STAGES - 1, (j + STAGES - 1) % STAGES);
            wait_vmem_n<2 * NLOAD * (STAGES - 1)>();
        } else {
            wait_vmem();
        }
        compute(j % STAGES, (t_begin + j) * BN);
    }

    // ---- epilogue
    const float l_tot = xhalf_sum((l_part[0] + l_part[1]) + (l_part[2] + l_part[3]));
    const float w_tot = xhalf_sum((w_part[0] + w_part[1]) + (w_part[2] + w_part[3]));
    const bool live = l_tot > 0.f;
    const float inv = live ? (KV8 ? p.vscale : 1.f) / w_tot : 0.f;
    const float lse_val = live ? (m_run + __log2f(l_tot)) * kLn2 : -__builtin_inff();
    const int64_t grow = (qtok0 + ti) * p.Hq + hh;
    if (!row_valid) return;
    // output slots 4q .. 4q+3 of block cb hold columns 32*cb + col4(q) + 0..3:
    // the bf16 transposing reads give A row m the column with bits 2 and 3
    // of m exchanged, the fp8 transposing reads column m itself
    auto col4 = [&](int q) { return KV8 ? 8 * q + 4 * half : 16 * (q >> 1) + 8 * half + 4 * (q & 1); };
    if (!SPLIT) {
        uint16_t* orow = p.o + grow * D;
#pragma unroll
        for (int cb = 0; cb < D / 32; ++cb) {
            if (KV8) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    bf16x4 ov;
#pragma unroll
                    for (int i = 0; i < 4; ++i) ov[i] = (__bf16)(oacc[cb][q * 4 + i] * inv);
                    *(bf16x4*)(orow + cb * 32 + col4(q)) = ov;
                }
            } else {  // two adjacent runs per 16-byte store
#pragma unroll
                for (int run = 0; run < 2; ++run) {
                    bf16x8 ov;
#pragma unroll
                    for (int i = 0; i < 8; ++i) ov[i] = (__bf16)(oacc[cb][run * 8 + i] * inv);
                    *(bf16x8*)(orow + cb * 32 + col4(2 * run)) = ov;
                }
            }
        }
        if (half == 0 && p.lse) p.lse[lse_index(p, b, hh, qtok0, ti, VARLEN)] = lse_val;
    } else {
        const int64_t rows = VARLEN ? (int64_t)p.total_q * p.Hq : (int64_t)p.B * p.Sq * p.Hq;
        float* orow = p.opart + ((int64_t)s * rows + grow) * D;
#pragma unroll
        for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                f32x4 v;
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = oacc[cb][q * 4 + i] * inv;
                *(f32x4*)(orow + cb * 32 + col4(q)) = v;
            }
        if (half == 0) {
            p.lpart[(int64_t)s * rows + grow] = lse_val;
            p.wpart[(int64_t)s * rows + grow] = live ? (m_run + __log2f(w_tot)) * kLn2 : -__builtin_inff();
        }
    }
}

// Merge of split partials. Split s wrote its output O_s, normalised by the
// sum of the bf16 probabilities it applied, the log-sum W_s of those
// probabilities and the log-sum-exp LSE_s of its fp32 probabilities. Then
//   O = sum_s exp(W_s - Mw) O_s / sum_s exp(W_s - Mw),   Mw = max_s W_s,
//   LSE = M + ln sum_s exp(LSE_s - M),                   M = max_s LSE_s,
// which is the unsplit normalisation of O and the unsplit LSE. A row whose
// splits are all empty gets O = 0 and LSE = -inf; a row whose keys all lie in
// one split gets that split's O and LSE unchanged. One row per D/4 lanes, 4
// columns a lane. The loops over the splits are unrolled so that eight loads
// are in flight at once (with few rows and many splits, as in single-sequence
// decode, the kernel is bound by load latency); the sums keep their split
// order.
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(const CombineParams p) {
    constexpr int LPR = D / 4;
    constexpr int RPB = 256 / LPR;
    const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
    const int c4 = threadIdx.x % LPR;
    if (row >= p.rows || !row_written(p, row)) return;
    float M = -__builtin_inff(), Mw = -__builtin_inff();
#pragma unroll 8
    for (int s = 0; s < p.ns; ++s) {
        M = fmaxf(M, p.lpart[(int64_t)s * p.rows + row]);
        Mw = fmaxf(Mw, p.wpart[(int64_t)s * p.rows + row]);
    }
    f32x4 acc = f32x4{};
    float lse = -__builtin_inff();
    if (M != -__builtin_inff()) {
        float tot = 0.f, totw = 0.f;
#pragma unroll 8
        for (int s = 0; s < p.ns; ++s) {
            tot += __expf(p.lpart[(int64_t)s * p.rows + row] - M);
            const float w = __expf(p.wpart[(int64_t)s * p.rows + row] - Mw);  // 0 for empty splits
            const f32x4 v = *(const f32x4*)(p.opart + ((int64_t)s * p.rows + row) * D + c4 * 4);
            totw += w;
            acc += w * v;
        }
        lse = M + __logf(tot);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = acc[i] / totw;
    }
    bf16x4 ov;
#pragma unroll
    for (int i = 0; i < 4; ++i) ov[i] = (__bf16)acc[i];
    *(bf16x4*)(p.o + row * D + c4 * 4) = ov;
    if (c4 == 0 && p.lse) p.lse[lse_row(p, row)] = lse;
}

// Many splits (single-sequence decode against a long context takes up to
// 128): one workgroup of 256 threads per row. Thread t takes columns
// 4*(t % (D/4)) .. +3 of the splits s = t / (D/4) + k*SG (SG split groups),
// so a row's ns partials are read SG at a time instead of one after the
// other; the groups' maxima, sums and weighted sums are merged through LDS.
// Same merge as combine_kernel (the sums run in another order).
template <int D>
__global__ __launch_bounds__(256) void combine_wide_kernel(const CombineParams p) {
    constexpr int LPR = D / 4;    // lanes per split group (4 columns each)
    constexpr int SG = 256 / LPR; // split groups
    __shared__ float sm_max[SG], sm_maxw[SG];
    __shared__ float sm_tot[SG], sm_totw[SG];
    __shared__ f32x4 sm_acc[SG][LPR];
    const int64_t row = blockIdx.x;
    if (row >= p.rows || !row_written(p, row)) return;  // uniform over the workgroup
    const int c4 = threadIdx.x % LPR, sg = threadIdx.x / LPR;
    float m = -__builtin_inff(), mw = -__builtin_inff();
#pragma unroll 4
    for (int s = sg; s < p.ns; s += SG) {
        m = fmaxf(m, p.lpart[(int64_t)s * p.rows + row]);
        mw = fmaxf(mw, p.wpart[(int64_t)s * p.rows + row]);
    }
    if (c4 == 0) {
        sm_max[sg] = m;
        sm_maxw[sg] = mw;
    }
    __syncthreads();
    float M = -__builtin_inff(), Mw = -__builtin_inff();
#pragma unroll
    for (int k = 0; k < SG; ++k) {
        M = fmaxf(M, sm_max[k]);
        Mw = fmaxf(Mw, sm_maxw[k]);
    }
    float tot = 0.f, totw = 0.f;
    f32x4 acc = f32x4{};
    if (M != -__builtin_inff()) {
#pragma unroll 4
        for (int s = sg; s < p.ns; s += SG) {
            tot += __expf(p.lpart[(int64_t)s * p.rows + row] - M);
            const float w = __expf(p.wpart[(int64_t)s * p.rows + row] - Mw);  // 0 for empty splits
            const f32x4 v = *(const f32x4*)(p.opart + ((int64_t)s * p.rows + row) * D + c4 * 4);
            totw += w;
            acc += w * v;
        }
    }
    if (c4 == 0) {
        sm_tot[sg] = tot;
        sm_totw[sg] = totw;
    }
    sm_acc[sg][c4] = acc;
    __syncthreads();
    if (sg != 0) return;
    float T = 0.f, Tw = 0.f;
    f32x4 A = f32x4{};
#pragma unroll
    for (int k = 0; k < SG; ++k) {
        T += sm_tot[k];
        Tw += sm_totw[k];
        A += sm_acc[k][c4];
    }
    const bool live = M != -__builtin_inff();
    bf16x4 ov;
#pragma unroll
    for (int i = 0; i < 4; ++i) ov[i] = (__bf16)(live ? A[i] / Tw : 0.f);
    *(bf16x4*)(p.o + row * D + c4 * 4) = ov;
    if (c4 == 0 && p.lse) p.lse[lse_row(p, row)] = live ? M + __logf(T) : -__builtin_inff();
}

// ---------------------------------------------------------------- launchers
template <int D, bool CAUSAL, bool SPLIT, bool VARLEN, bool QK8, bool PAGED>
static hipError_t launch_attn(const FwdParams& p, hipStream_t stream) {
    hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL, SPLIT, VARLEN, QK8, PAGED>), dim3(p.grid), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

template <int D, bool VARLEN, bool QK8, bool PAGED>
static hipError_t launch_attn_d(const FwdParams& p, bool causal, bool split, hipStream_t stream) {
    if (causal)
        return split ? launch_attn<D, true, true, VARLEN, QK8, PAGED>(p, stream)
                     : launch_attn<D, true, false, VARLEN, QK8, PAGED>(p, stream);
    return split ? launch_attn<D, false, true, VARLEN, QK8, PAGED>(p, stream)
                 : launch_attn<D, false, false, VARLEN, QK8, PAGED>(p, stream);
}

// Instantiated combinations: bf16, variable-length bf16, fp8 Q/K, paged bf16.
template <int D>
static hipError_t launch_attn_dd(const FwdParams& p, bool causal, bool split, bool varlen, bool qk8, bool paged,
                                 hipStream_t stream) {
    if (qk8) return launch_attn_d<D, false, true, false>(p, causal, split, stream);
    if (paged) return launch_attn_d<D, false, false, true>(p, causal, split, stream);
    return varlen ? launch_attn_d<D, true, false, false>(p, causal, split, stream)
                  : launch_attn_d<D, false, false, false>(p, causal, split, stream);
}

hipError_t launch_attention(const FwdParams& p, int d, bool causal, bool split, bool varlen, bool qk8, bool paged,
                            hipStream_t stream) {
    return d == 128 ? launch_attn_dd<128>(p, causal, split, varlen, qk8, paged, stream)
                    : launch_attn_dd<64>(p, causal, split, varlen, qk8, paged, stream);
}

template <bool CAUSAL, bool PAGED, bool VARLEN, bool QK8 = false>
static void launch_pp(const FwdParams& p, hipStream_t stream) {
    hipLaunchKernelGGL((attn_fwd_pingpong_kernel<128, CAUSAL, PAGED, VARLEN, QK8>), dim3(p.grid), dim3(kPPThreads), 0,
                       stream, p);
}

// d=128 only (the plan never picks this kernel at d=64)
hipError_t launch_pingpong(const FwdParams& p, int d, bool causal, bool paged, bool varlen, bool qk8,
                           hipStream_t stream) {
    if (d != 128 || (paged && varlen) || (qk8 && (paged || varlen))) return hipErrorInvalidValue;
    if (qk8) causal ? launch_pp<true, false, false, true>(p, stream) : launch_pp<false, false, false, true>(p, stream);
    else if (paged) causal ? launch_pp<true, true, false>(p, stream) : launch_pp<false, true, false>(p, stream);
    else if (varlen) causal ? launch_pp<true, false, true>(p, stream) : launch_pp<false, false, true>(p, stream);
    else causal ? launch_pp<true, false, false>(p, stream) : launch_pp<false, false, false>(p, stream);
    return hipGetLastError();
}

template <int D, bool CAUSAL, bool SPLIT, bool PAGED, bool KV8, bool VARLEN>
static hipError_t launch_dec(const FwdParams& p, hipStream_t stream) {
    hipLaunchKernelGGL((attn_decode_kernel<D, CAUSAL, SPLIT, PAGED, KV8, VARLEN, KV8 ? kDecStagesKV8 : kDecStages>),
                       dim3(p.grid), dim3(kDecThreads), 0, stream, p);
    return hipGetLastError();
}

template <int D, bool PAGED, bool KV8, bool VARLEN>
static hipError_t launch_dec_d(const FwdParams& p, bool causal, bool split, hipStream_t stream) {
    if (causal)
        return split ? launch_dec<D, true, true, PAGED, KV8, VARLEN>(p, stream)
                     : launch_dec<D, true, false, PAGED, KV8, VARLEN>(p, stream);
    return split ? launch_dec<D, false, true, PAGED, KV8, VARLEN>(p, stream)
                 : launch_dec<D, false, false, PAGED, KV8, VARLEN>(p, stream);
}

// Instantiated combinations: contiguous, paged, fp8, paged fp8, variable-length (bf16).
template <int D>
static hipError_t launch_dec_dd(const FwdParams& p, bool causal, bool split, bool paged, bool kv8, bool varlen,
                                hipStream_t stream) {
    if (varlen) return launch_dec_d<D, false, false, true>(p, causal, split, stream);
    if (paged)
        return kv8 ? launch_dec_d<D, true, true, false>(p, causal, split, stream)
                   : launch_dec_d<D, true, false, false>(p, causal, split, stream);
    return kv8 ? launch_dec_d<D, false, true, false>(p, causal, split, stream)
               : launch_dec_d<D, false, false, false>(p, causal, split, stream);
}

hipError_t launch_decode(const FwdParams& p, int d, bool causal, bool split, bool paged, bool kv8, bool varlen,
                         hipStream_t stream) {
    return d == 128 ? launch_dec_dd<128>(p, causal, split, paged, kv8, varlen, stream)
                    : launch_dec_dd<64>(p, causal, split, paged, kv8, varlen, stream);
}

hipError_t launch_combine(const CombineParams& p, int d, long long grid, hipStream_t stream) {
    if (p.ns >= kCombineWideSplits) {  // one workgroup per row (grid == rows)
        if (d == 128)
            hipLaunchKernelGGL((combine_wide_kernel<128>), dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
        else
            hipLaunchKernelGGL((combine_wide_kernel<64>), dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
        return hipGetLastError();
    }
    if (d == 128)
        hipLaunchKernelGGL((combine_kernel<128>), dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((combine_kernel<64>), dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace gqa
