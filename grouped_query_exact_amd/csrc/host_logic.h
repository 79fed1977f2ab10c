// Host-side logic of the GQA forward library: argument checks, the
// pack/split heuristic, launch planning and the magic-number divisor.
// Plain C++ with no HIP calls, so it can be built and tested on a CPU.
#pragma once

#include <cstdint>

namespace gqa {

// Tile shape of the attention kernel: 4 wavefronts of 64 lanes, each owning
// 32 query rows, stream 64 keys per step.
constexpr int kBlockM = 128;
constexpr int kBlockN = 64;
constexpr int kThreads = 256;

// Large unsplit bf16 prefill launches at d=128 (at d=64 the 4-wavefront
// kernel fits four wavefronts per SIMD and is as fast or faster, measured):
// 8 wavefronts own 256 packed rows and
// a compute unit, in two groups that alternate between matrix products and
// softmax, with a ring of kPPStages K/V stages (128 KiB of LDS at d=128).
// Chosen when the call has at least kPPMinItemsPerCU such work items per
// compute unit, or one per compute unit with kPPMinKeyTiles key tiles per
// item on average; smaller grids keep the 4-wavefront kernel, two per CU.
constexpr int kPPBlockM = 256;
constexpr int kPPThreads = 512;
constexpr int kPPStages = 4;
constexpr int kPPMinItemsPerCU = 2;
constexpr int kPPMinKeyTiles = 32;

// Decode-shaped launches (at most kDecBlockM query rows per head unit, e.g.
// one new token of a KV group): one wavefront per workgroup streaming tiles
// of kDecBlockN keys through a ring of kDecStages LDS stages.
constexpr int kDecBlockM = 32;
constexpr int kDecBlockN = 32;
constexpr int kDecThreads = 64;
constexpr int kDecStages = 4;
// fp8 K/V: half the bytes per stage (32 KiB per workgroup at d=128); 6 and
// 8 stages measured no faster.
constexpr int kDecStagesKV8 = 4;

// Backward pass: the dK/dV kernel takes 128 keys per workgroup of
// kBwdThreads (32 keys per wavefront, one wavefront for dK and one for dV)
// against query tiles of kBwdRows packed rows, streamed through a ring of
// kBwdStages LDS stages (tiles j-1 and j in use, kBwdStages - 2 in flight).
constexpr int kBwdKeys = 128;
constexpr int kBwdRows = 64;
constexpr int kBwdThreads = 512;
constexpr int kBwdStages = 3;

// Division by a runtime constant through a precomputed multiplier (the
// batch-sensitivity article, "PackGQA" mechanism 3, precomputes the
// query-head -> KV-head map with a fast divide-and-modulo). Round-up method:
// with l = ceil(log2 d) and m = floor(2^32 * (2^l - d) / d) + 1,
// n / d == (umulhi(n, m) + n) >> l for every 0 <= n < 2^31.
struct FastDiv {
    uint32_t div;
    uint32_t mul;
    uint32_t shift;
};
FastDiv make_fastdiv(uint32_t d);
inline uint32_t fastdiv_host(uint32_t n, const FastDiv& f) {
    uint32_t hi = (uint32_t)(((uint64_t)n * f.mul) >> 32);
    return (hi + n) >> f.shift;
}

struct Shape {
    int B, Sq, Sk, Hq, Hk, d, causal;
    int kv_bytes = 2;  // bytes per stored K/V element: 2 (bf16) or 1 (fp8)
    int q_bytes = 2;   // bytes per stored Q element: 2 (bf16) or 1 (fp8 Q and K)
    int varlen = 0;    // packed sequences of different lengths (Sq, Sk: the bounds max_seqlen_q, max_seqlen_k)
    long long total_q = 0;  // variable-length calls: query tokens of all sequences
    int paged = 0;     // K/V in a pool of pages
};

// Returns 0 or a gqa_status_t error for the sizes alone (no pointers).
int check_sizes(const Shape& s, float scale, int pack_gqa, int num_splits);

// The heuristic: resolves pack_gqa (0/1) and num_splits (>= 1).
void choose(const Shape& s, int num_cus, int* pack_gqa, int* num_splits);

struct Plan {
    int decode;         // 1: decode kernel (R <= kDecBlockM), 0: tiled kernel
    int pingpong;       // 1: the 8-wavefront tiled kernel (kPPBlockM rows), 0: 4 wavefronts
    int worklist;       // variable-length prefill: items from the scheduling kernel's work list
    int pair_rows;      // causal batched 8-wavefront launches: two mirrored row tiles per workgroup
    int threads;        // threads per attention workgroup
    int block_m;        // query rows per tile
    int block_n;        // keys per tile
    int pack;           // resolved pack flag
    int G;              // query heads per KV head
    int Gp;             // rows per token in a tile: G if packed, else 1
    int units_per_b;    // head units per batch element: Hk if packed, else Hq
    long long R;        // query rows per head unit: Sq * Gp
    int row_tiles;      // ceil(R / block_m)
    int key_tiles;      // key tiles of the longest row tile
    int ns;             // resolved, clamped split count
    long long grid;     // attention workgroups
    long long combine_grid;
    long long workspace_bytes;
};

// Resolves the plan; returns 0 or a status (sizes too large for the grid).
int make_plan(const Shape& s, int pack_gqa, int num_splits, int num_cus, Plan* p);

// Rows of the combine kernel handled by one 256-thread workgroup. From
// kCombineWideSplits splits on, the merge takes one workgroup per row, whose
// threads share out the splits.
inline int combine_rows_per_block(int d) { return kThreads / (d / 4); }
constexpr int kCombineWideSplits = 16;

// Fixed split-KV workspace of gqa_attn_fwd_noalloc (a file-scope device array,
// one copy per GPU): 64 MiB holds the partials of every decode-shaped call up
// to B*Hq = 4096 query rows at 8 splits (d=128), or 32 splits of 1024 rows.
constexpr long long kScratchBytes = 64LL << 20;

}  // namespace gqa
