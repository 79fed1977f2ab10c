// Host-side logic: argument checks, heuristic, launch plan, magic divisor.
#include "host_logic.h"

#include <algorithm>
#include <climits>
#include <cmath>

#include "../../include/gqa_attn.h"

namespace gqa {

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

// Key tiles needed by the row tile holding query rows [r0, r1) of a head unit.
static int key_tiles_for(const Shape& s, int Gp, long long r0, long long r1) {
    long long kv_end = s.Sk;
    if (s.causal) {
        long long i_max = (r1 - 1) / Gp;
        kv_end = std::min<long long>(s.Sk, i_max + (s.Sk - s.Sq) + 1);
    }
    if (kv_end <= 0) return 0;
    (void)r0;
    return (int)ceil_div(kv_end, kBlockN);
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

    // Split the keys when the grid is too small to fill the GPU. A workgroup
    // that owns only a few query rows is memory-bound (decode): it then needs
    // many more workgroups in flight to cover HBM latency.
    const int Gp = pack ? G : 1;
    const long long R = (long long)s.Sq * Gp;
    const long long units = (long long)s.B * (pack ? s.Hk : s.Hq) * ceil_div(R, kBlockM);
    const int T = key_tiles_for(s, Gp, std::max<long long>(0, R - kBlockM), R);
    const bool memory_bound = R <= kBlockM / 4;
    const long long target = (memory_bound ? 8LL : 2LL) * num_cus;
    int ns = 1;
    if (units > 0 && units < target && T > 1) {
        ns = (int)std::min<long long>(ceil_div(target, units), 16);
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
    p->row_tiles = (int)ceil_div(p->R, kBlockM);
    p->key_tiles = p->R > 0 ? key_tiles_for(s, p->Gp, std::max<long long>(0, p->R - kBlockM), p->R) : 0;
    ns = std::max(1, std::min(ns, std::max(1, p->key_tiles)));
    p->ns = ns;
    p->grid = (long long)s.B * p->units_per_b * p->row_tiles * ns;
    if (p->grid > INT_MAX) return GQA_ERR_INVALID_ARG;
    const long long rows = (long long)s.B * s.Sq * s.Hq;
    if (ns > 1) {
        p->combine_grid = ceil_div(rows, combine_rows_per_block(s.d));
        p->workspace_bytes = (long long)ns * rows * ((long long)s.d * 4 + 4);
        if (p->combine_grid > INT_MAX) return GQA_ERR_INVALID_ARG;
    } else {
        p->combine_grid = 0;
        p->workspace_bytes = 0;
    }
    return GQA_OK;
}

}  // namespace gqa
