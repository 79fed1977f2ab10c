// Kernel parameter blocks and launchers of the GQA forward library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "host_logic.h"

namespace gqa {

struct FwdParams {
    const uint16_t* q;  // [B, Sq, Hq, D] bf16
    const uint16_t* k;  // [B, Sk, Hk, D] bf16
    const uint16_t* v;  // [B, Sk, Hk, D] bf16
    uint16_t* o;        // [B, Sq, Hq, D] bf16 (unsplit launches)
    float* lse;         // [B, Hq, Sq] fp32 or null (unsplit launches)
    float* opart;       // [ns, B*Sq*Hq, D] fp32 (split launches): O_s, normalised by its bf16 weights
    float* lpart;       // [ns, B*Sq*Hq] fp32 (split launches): LSE_s of the fp32 probabilities
    float* wpart;       // [ns, B*Sq*Hq] fp32 (split launches): log-sum of the bf16 probabilities
    int B, Sq, Sk, Hq, Hk;
    int G;              // Hq / Hk
    int Gp;             // rows per token in a tile: G when packed, 1 otherwise
    uint32_t gmul, gshift;  // magic divisor of Gp
    int R;              // query rows per head unit: Sq * Gp
    int row_tiles;      // ceil(R / rows per tile)
    int units_per_b;    // Hk when packed, Hq otherwise
    int ns;             // key splits
    int grid;           // workgroups
    int pair_rows;      // causal 8-wavefront launches: 1 = two row tiles (rt, row_tiles-1-rt) per workgroup
    float c;            // |scale| * log2(e), or 1 when scale == 0
    uint32_t qand;      // 0 when scale == 0 (Q read as zeros: every visible score is 0), else all ones
    uint32_t qsign;     // sign bits that negate Q (negative score factor): 0x80008000 bf16, 0x80808080 fp8; else 0
    // paged K/V (decode kernel only): k and v point at page pools
    // [num_pages, page_size, Hk, D]; Sk is unused.
    const int* block_table;  // [B, max_pages] pool page of each logical page
    const int* seqlens_k;    // [B] keys of each sequence
    int page_size, max_pages, num_pages;
    uint32_t pmul, pshift;   // magic divisor of page_size
    float vscale;            // fp8 K/V (decode kernel): factor of the values
    // variable-length calls: q/o [total_q, Hq, D], k/v [total_k, Hk, D], lse
    // [Hq, total_q]; Sq is max_seqlen_q (the grid's row tiles), Sk unused.
    const int* cu_q;         // [B+1] cumulative query lengths
    const int* cu_k;         // [B+1] cumulative key lengths
    int total_q, total_k;
    // variable-length calls on the tiled kernel: the work list the scheduling
    // kernel wrote (count, then (sequence, row tile) pairs, heaviest first);
    // workgroup i takes pair (i / ns) / units_per_b, head unit (i / ns) % units_per_b
    const int* worklist;
};

// The scheduling kernel of variable-length prefill (one workgroup).
struct SchedParams {
    const int* cu_q;
    const int* cu_k;
    int* worklist;           // [1 + 2 * cap]: count, then (b, rt) entries (pair mode: (b, pr))
    int B, total_q, total_k, max_sq, Gp;
    uint32_t gmul, gshift;   // magic divisor of Gp
    int block_m;             // rows per tile of the attention kernel
    int causal;
    int pair;                // 1: an entry is (b, pr), row tiles R_b-1-pr and pr of sequence b together
    int cap;                 // entries the list can hold
};
hipError_t launch_schedule(const SchedParams& sp, hipStream_t stream);
constexpr int kSchedThreads = 1024;
constexpr int kSchedBins = 1024;  // cost bins (key tiles), the last one collects longer items

struct CombineParams {
    const float* opart;
    const float* lpart;
    const float* wpart;
    uint16_t* o;
    float* lse;
    int64_t rows;       // B * Sq * Hq (variable-length calls: total_q * Hq)
    int ns, Sq, Hq;     // variable-length calls: Sq = total_q (LSE [Hq, total_q])
    // variable-length calls: the rows the attention kernel wrote are the first
    // min(length, max_sq) tokens of each sequence; the combine skips the others
    const int* cu_q;    // [B+1] cumulative query lengths, or null (every row written)
    int B, total_q, max_sq;
};

// Backward pass (always PackGQA rows: the G query heads of a KV group).
struct BwdParams {
    const uint16_t* q;     // [B, Sq, Hq, D] bf16
    const uint16_t* k;     // [B, Sk, Hk, D]
    const uint16_t* v;     // [B, Sk, Hk, D]
    const uint16_t* o;     // [B, Sq, Hq, D] forward output
    const uint16_t* dout;  // [B, Sq, Hq, D] upstream gradient
    const float* lse;      // [B, Hq, Sq] forward log-sum-exp (natural log)
    float* drow;           // [B, Hq, Sq] workspace: D = rowsum(dO * O)
    float* nlse2;          // [B, Hq, Sq] workspace: -LSE * log2(e), -inf for rows without keys
    uint16_t* dq;          // [B, Sq, Hq, D]
    uint16_t* dk;          // [B, Sk, Hk, D]
    uint16_t* dv;          // [B, Sk, Hk, D]
    int B, Sq, Sk, Hq, Hk, G;
    uint32_t gmul, gshift; // magic divisor of G
    int R;                 // packed rows per KV group: Sq * G
    int row_tiles;         // dQ kernel: ceil(R / kBlockM)
    int key_blocks;        // dK/dV kernel: ceil(Sk / kBwdKeys)
    int grid_dq, grid_dkdv;
    float c;               // scale * log2(e), with the sign of scale
    float scale;
};

hipError_t launch_backward(const BwdParams& p, int d, bool causal, hipStream_t stream);

hipError_t launch_attention(const FwdParams& p, int d, bool causal, bool split, bool varlen, bool qk8, bool paged,
                            hipStream_t stream);
// unsplit bf16 prefill on the 8-wavefront kernel (p.row_tiles of kPPBlockM rows)
hipError_t launch_pingpong(const FwdParams& p, int d, bool causal, bool paged, bool varlen, bool qk8,
                           hipStream_t stream);
hipError_t launch_decode(const FwdParams& p, int d, bool causal, bool split, bool paged, bool kv8, bool varlen,
                         hipStream_t stream);
hipError_t launch_combine(const CombineParams& p, int d, long long grid, hipStream_t stream);

// Device address of the fixed workspace on device `dev` (the current device),
// looked up once per device (gqa_attn_scratch.hip).
hipError_t scratch_address(int dev, void** ptr);

}  // namespace gqa
