// Host-side logic: argument checks, heuristic, launch plan, magic divisor.
#include "host_logic.h"

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdlib>

#include "../../include/gqa_attn.h"

namespace gqa {

// fewest key tiles per row for a non-causal batched call on the 8-wavefront kernel
constexpr int kPPMinKeyTilesNonCausal = 9;

FastDiv make_fastdiv(uint32_t d) {
    FastDiv f{d, 0, 0};
    uint32_t l = 0;
    while (l < 32 && (1ull << l) < d) ++l;
    f.shift = l;
    f.mul = (uint32_t)(((1ull << 32) * ((1ull << l) - d)) / d + 1);
    return f;
}

int check_sizes(const Shape& s, float scale, int pack_gqa, int num_splits) {
    if (s.B < 0 || s.Sq < 0 || s.Sk < 0 || s.Hq <= 0 || s.Hk <= 0) return GQA_ERR_INVALID_ARG;
    if (s.Hq % s.Hk != 0) return GQA_ERR_INVALID_ARG;
    if (pack_gqa < -1 || pack_gqa > 1) return GQA_ERR_INVALID_ARG;
    if (num_splits < 0) return GQA_ERR_INVALID_ARG;
    if (!std::isfinite(scale)) return GQA_ERR_INVALID_ARG;
    if ((long long)s.B * s.Sq > 0 && s.Sk == 0) return GQA_ERR_INVALID_ARG;
    if (s.d != 64 && s.d != 128) return GQA_ERR_UNSUPPORTED;
    return GQA_OK;
}

static long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }

// Key tiles (of bn keys) needed by the last row of a tile ending at row r1
// of a head unit.
static int key_tiles_for(const Shape& s, int Gp, long long r1, int bn) {
    long long kv_end = s.Sk;
    if (s.causal) {
        long long i_max = (r1 - 1) / Gp;
        kv_end = std::min<long long>(s.Sk, i_max + (s.Sk - s.Sq) + 1);
    }
    if (kv_end <= 0) return 0;
    return (int)ceil_div(kv_end, bn);
}

void choose(const Shape& s, int num_cus, int* pack_gqa, int* num_splits) {
    const int G = s.Hq / s.Hk;
    if (num_cus <= 0) num_cus = 256;
    // Pack when it fills the tiles at least as well: the rows of one head
    // (Sq) against the rows of one group (Sq*G). Packing also narrows the
    // causal band a tile spans (fewer tokens per tile), and in decode it
    // reads each K/V tile once per group instead of once per query head.
    const long long tiles_np = ceil_div(s.Sq, kBlockM);
    const long long tiles_p = ceil_div((long long)s.Sq * G, kBlockM);
    const double util_np = tiles_np ? (double)s.Sq / (tiles_np * kBlockM) : 0.0;
    const double util_p = tiles_p ? (double)s.Sq * G / (tiles_p * kBlockM) : 0.0;
    const int pack = (G > 1 && util_p >= util_np) ? 1 : 0;
    *pack_gqa = pack;

    // Split the keys when the grid is too small to fill the GPU. The tiled
    // kernel wants two workgroups per compute unit. The bf16 decode kernel
    // (at most 32 rows, memory-bound, kDecStages-1 tiles in flight per
    // workgroup) is split only up to one workgroup per compute unit: measured
    // on MI355X from one sequence against 128K keys to 64 sequences against
    // 8K, that count is the fastest, and more, shorter workgroups add tail and
    // merge costs (a single sequence needs up to 32 splits for it). With fp8
    // K/V a tile costs more arithmetic per byte (the conversion to bf16):
    // two workgroups per compute unit are fastest when each unit has at
    // least 256 key tiles to stream and there are at least 32 head units
    // (64 x 8K, 8 x 32K, 4 x 64K keys: 9-13% faster than four), four
    // otherwise (one sequence against 128K keys: 52 us at 128 splits, 57 at
    // 64; against 256K keys 108 us at 128, 117 at 64; 32 x 4K keys), up to
    // 128 splits.
    const int Gp = pack ? G : 1;
    const long long R = (long long)s.Sq * Gp;
    const bool decode = R <= kDecBlockM && s.q_bytes == 2;
    const int bm = decode ? kDecBlockM : kBlockM, bn = decode ? kDecBlockN : kBlockN;
    const long long units = (long long)s.B * (pack ? s.Hk : s.Hq) * ceil_div(R, bm);
    const int T = R > 0 ? key_tiles_for(s, Gp, R, bn) : 0;
    const bool dec16 = decode && s.kv_bytes == 2;
    const long long per_cu = !decode ? 2 : dec16 ? 1 : (units >= 32 && units * T >= 256LL * num_cus ? 2 : 4);
    const long long target = per_cu * num_cus;
    const int cap = decode ? (dec16 ? 64 : 128) : 16;
    int ns = 1;
    if (units > 0 && units < target && T > 1) {
        ns = (int)std::min<long long>(ceil_div(target, units), cap);
        ns = std::max(1, std::min(ns, T / 2 > 0 ? T / 2 : 1));
    }
    *num_splits = ns;
}

int make_plan(const Shape& s, int pack_gqa, int num_splits, int num_cus, Plan* p) {
    int pack = pack_gqa, ns = num_splits;
    if (pack < 0 || ns == 0) {
        int cp = 0, cn = 1;
        choose(s, num_cus, &cp, &cn);
        if (pack < 0) pack = cp;
        if (ns == 0) ns = cn;
    }
    const int G = s.Hq / s.Hk;
    if (G == 1) pack = 0;  // one head per group: packing is the same tiling
    p->pack = pack;
    p->G = G;
    p->Gp = pack ? G : 1;
    p->units_per_b = pack ? s.Hk : s.Hq;
    p->R = (long long)s.Sq * p->Gp;
    if (p->R > INT_MAX / 2) return GQA_ERR_INVALID_ARG;
    p->decode = p->R <= kDecBlockM && s.q_bytes == 2 ? 1 : 0;
    p->block_m = p->decode ? kDecBlockM : kBlockM;
    p->block_n = p->decode ? kDecBlockN : kBlockN;
    p->row_tiles = (int)ceil_div(p->R, p->block_m);
    p->key_tiles = p->R > 0 ? key_tiles_for(s, p->Gp, p->R, p->block_n) : 0;
    ns = std::max(1, std::min(ns, std::max(1, p->key_tiles)));
    p->ns = ns;
    // Unsplit bf16 calls at d=128 with enough 256-row items to give every
    // compute unit kPPMinItemsPerCU of them run on the 8-wavefront kernel
    // (or one per compute unit when the items are long: an estimated average
    // of at least kPPMinKeyTiles key tiles, from the first and last row
    // tile). Variable-length calls count the items their tokens fill and take
    // that kernel only from a work list (on the plain grid the empty items
    // cost it more: 683 TFLOP/s on it against 730 on the 4-wavefront kernel
    // for 16 sequences of 128..2048 tokens). GQA_ATTN_FORCE_TILED=1 in the
    // environment keeps every prefill call on the 4-wavefront kernel (same
    // results bit for bit; for comparisons).
    const char* force_env = std::getenv("GQA_ATTN_FORCE_TILED");
    const bool force_tiled = force_env && force_env[0] && !(force_env[0] == '0' && !force_env[1]);
    // fp8 Q/K calls (q_bytes == 1) take it for contiguous batched calls
    const bool pp_qk = s.q_bytes == 2 || (s.q_bytes == 1 && !s.varlen && !s.paged);
    const bool pp_shape = !force_tiled && !p->decode && ns == 1 && s.d == 128 && pp_qk && s.kv_bytes == 2;
    const long long cus = num_cus > 0 ? num_cus : 256;
    const bool pp_varlen = pp_shape && s.varlen &&
                           p->units_per_b * (ceil_div(s.total_q * p->Gp, kPPBlockM) + s.B) >= (long long)kPPMinItemsPerCU * cus;
    // Variable-length prefill runs from a work list that a scheduling kernel
    // builds on the device (only the (sequence, row tile) items that exist,
    // heaviest first) when its sequences leave most of the grid empty (fewer
    // than 3/4 of B * max_seqlen_q query tokens), and always when it goes to
    // the 8-wavefront kernel. Measured on MI355X, Llama-2 heads: for about
    // full batches the 4-wavefront kernel's plain grid beats the list on the
    // same kernel (8 x 2048 tokens, causal: 855 against 801 TFLOP/s), but the
    // list on the 8-wavefront kernel beats both (8 x 2048, 12 sequences of
    // 1500..1900 tokens, 16 x 1000, 32 x 512, 4 x 4096: causal 910, 865,
    // 745, 539, 1026 against 857, 802, 715, 485, 967 from the grid;
    // non-causal 1042, 997, 897, 756, 1124 against 928, 823, 817, 641, 989).
    p->worklist = s.varlen && !p->decode && (4 * s.total_q < 3LL * s.B * s.Sq || pp_varlen) ? 1 : 0;
    p->pingpong = 0;
    // Non-causal batched calls whose rows read at most 8 key tiles keep the
    // 4-wavefront kernel: measured on MI355X, Llama-2 heads, it is 14% faster
    // at 384 keys and within +-5% at 512; the 8-wavefront kernel is 3-8%
    // faster from 768 keys on. Causal calls, whose row tiles the 8-wavefront
    // kernel pairs, take it at any length (6-9% faster down to 128 tokens).
    if (s.varlen) {
        p->pingpong = pp_varlen ? 1 : 0;
    } else if (pp_shape && (s.causal || p->key_tiles >= kPPMinKeyTilesNonCausal)) {
        const long long items = (long long)s.B * p->units_per_b * ceil_div(p->R, kPPBlockM);
        if (items >= (long long)kPPMinItemsPerCU * cus) {
            p->pingpong = 1;
        } else if (items >= cus) {
            const int first = key_tiles_for(s, p->Gp, std::min<long long>(p->R, kPPBlockM), kBlockN);
            const int last = key_tiles_for(s, p->Gp, p->R, kBlockN);
            if ((long long)first + last >= 2LL * kPPMinKeyTiles) p->pingpong = 1;
        }
    }
    if (p->pingpong) {
        p->block_m = kPPBlockM;
        p->row_tiles = (int)ceil_div(p->R, kPPBlockM);
    }
    p->threads = p->decode ? kDecThreads : (p->pingpong ? kPPThreads : kThreads);
    p->grid = (long long)s.B * p->units_per_b * p->row_tiles * ns;
    // causal launches of the 8-wavefront kernel pair each row tile with its
    // mirror (row_tiles-1-rt) in one workgroup: equal key tiles per workgroup,
    // and the light item's Q rows arrive while the heavy one finishes. Only
    // when the pairs still give every compute unit one: a chunk of new tokens
    // against a long cached context has few row tiles of nearly equal cost,
    // and pairing would leave half the GPU idle (measured on MI355X, 2048
    // tokens against 65536 keys, Llama-2 heads: 2.81 ms paired on 128
    // workgroups, 1.9-2.0 ms unpaired on 256).
    p->pair_rows = 0;
    if (p->pingpong && s.causal && !s.varlen) {
        const long long pairs = (long long)s.B * p->units_per_b * ((p->row_tiles + 1) / 2);
        if (pairs >= cus) {
            p->pair_rows = 1;
            p->grid = pairs;
        }
    }
    if (p->grid > INT_MAX) return GQA_ERR_INVALID_ARG;
    const long long rows = (long long)s.B * s.Sq * s.Hq;
    if (ns > 1) {
        p->combine_grid = ns >= kCombineWideSplits ? rows : ceil_div(rows, combine_rows_per_block(s.d));
        p->workspace_bytes = (long long)ns * rows * ((long long)s.d * 4 + 8);  // O_s, LSE_s, W_s (fp32)
        if (p->combine_grid > INT_MAX) return GQA_ERR_INVALID_ARG;
    } else {
        p->combine_grid = 0;
        p->workspace_bytes = 0;
    }
    return GQA_OK;
}

}  // namespace gqa
