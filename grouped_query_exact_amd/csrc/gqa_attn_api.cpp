// C-ABI entry points of the GQA forward library (declared in include/gqa_attn.h).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <utility>

#include "../../include/gqa_attn.h"
#include "host_logic.h"
#include "kernels.h"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];
std::once_flag g_pool_once[kMaxDevices];

int current_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return -1;
    return dev;
}

// Compute units of the current device, cached per device. 0 on failure.
int device_cus(int dev) {
    if (dev < 0 || dev >= kMaxDevices) return 0;
    int n = g_cu_count[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    g_cu_count[dev].store(v, std::memory_order_relaxed);
    return v;
}

// Split and backward workspaces come from a stream-ordered memory pool the
// library owns, one per device. It keeps up to kPoolKeepBytes reserved
// between calls, so steady-state calls (decode splits need a few MB) take
// nothing from the driver, and returns anything above that to the device at
// the next synchronisation (a 35 GB split workspace is not held for good).
// The device's default pool, which other code uses, is left as it is. If the
// pool cannot be created, the default pool serves the allocations.
constexpr uint64_t kPoolKeepBytes = 256ull << 20;
hipMemPool_t g_pool[kMaxDevices];

hipMemPool_t lib_pool(int dev) {
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    std::call_once(g_pool_once[dev], [dev] {
        hipMemPoolProps props = {};
        props.allocType = hipMemAllocationTypePinned;
        props.handleTypes = hipMemHandleTypeNone;
        props.location.type = hipMemLocationTypeDevice;
        props.location.id = dev;
        hipMemPool_t pool = nullptr;
        if (hipMemPoolCreate(&pool, &props) != hipSuccess || !pool) {
            (void)hipGetLastError();
            return;
        }
        uint64_t thr = kPoolKeepBytes;
        (void)hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &thr);
        g_pool[dev] = pool;
    });
    return g_pool[dev];
}

// Stream-ordered workspace allocation from the library's pool (see lib_pool).
hipError_t ws_alloc(void** ptr, size_t bytes, int dev, hipStream_t stream) {
    hipMemPool_t pool = lib_pool(dev);
    return pool ? hipMallocFromPoolAsync(ptr, bytes, pool, stream) : hipMallocAsync(ptr, bytes, stream);
}

// Workspaces of up to kWsCacheBytes are kept per (device, stream) and reused
// by later calls on that stream: calls on one stream run in order, so a
// buffer that only that stream's work uses needs no allocation, release or
// wait between them (a stream-ordered allocation and release per call left
// the GPU idle for several microseconds between the kernels of consecutive
// split decode calls). A call that needs more than the stream's buffer
// holds releases it after the work already enqueued on that stream and
// takes a larger one, stream-ordered. A call holds its stream's buffer
// (a lock of its own) from the lookup until its kernels are enqueued, so
// host threads that share a stream cannot release a buffer between another
// call's lookup and its launches. At most kWsCacheEntries streams get a
// kept buffer; calls on further streams, calls being captured into a graph
// and calls that need more than kWsCacheBytes allocate and release their
// workspace per call, as before. Kept buffers live until the process ends.
constexpr size_t kWsCacheBytes = 64ull << 20;
constexpr int kWsCacheEntries = 16;
struct WsEntry {
    int dev = -1;
    hipStream_t stream = nullptr;
    void* ptr = nullptr;
    size_t bytes = 0;
    std::mutex mu;  // held by the call using the buffer
};
std::mutex g_ws_mu;  // the table (lookup and insertion)
WsEntry g_ws[kWsCacheEntries];
int g_ws_used = 0;

// A call's workspace: a kept buffer (held through `hold` until the lease
// ends) or a per-call allocation (released by the caller with hipFreeAsync).
struct WsLease {
    void* ptr = nullptr;
    bool kept = false;
    std::unique_lock<std::mutex> hold;
};

// A workspace of `bytes` for work enqueued on `stream` of device `dev`.
hipError_t ws_acquire(size_t bytes, int dev, hipStream_t stream, WsLease* lease) {
    lease->ptr = nullptr;
    lease->kept = false;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cap) != hipSuccess) {
        (void)hipGetLastError();
        cap = hipStreamCaptureStatusActive;  // unknown: take the per-call path
    }
    if (bytes > kWsCacheBytes || cap != hipStreamCaptureStatusNone) return ws_alloc(&lease->ptr, bytes, dev, stream);
    WsEntry* e = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_ws_mu);
        for (int i = 0; i < g_ws_used; ++i)
            if (g_ws[i].dev == dev && g_ws[i].stream == stream) e = &g_ws[i];
        if (!e) {
            if (g_ws_used == kWsCacheEntries) return ws_alloc(&lease->ptr, bytes, dev, stream);
            e = &g_ws[g_ws_used];
            e->dev = dev;
            e->stream = stream;
            ++g_ws_used;
        }
    }
    std::unique_lock<std::mutex> hold(e->mu);
    if (e->bytes < bytes) {
        // grow in steps of 1 MiB, at least doubling, up to the cap
        size_t want = std::max(bytes, std::min(2 * e->bytes, kWsCacheBytes));
        want = (want + (1u << 20) - 1) & ~(size_t)((1u << 20) - 1);
        want = std::min(std::max(want, bytes), kWsCacheBytes);
        if (e->ptr && hipFreeAsync(e->ptr, stream) != hipSuccess) return hipErrorUnknown;
        e->ptr = nullptr;
        e->bytes = 0;
        void* fresh = nullptr;
        const hipError_t err = ws_alloc(&fresh, want, dev, stream);
        if (err != hipSuccess || !fresh) return err != hipSuccess ? err : hipErrorOutOfMemory;
        e->ptr = fresh;
        e->bytes = want;
    }
    lease->ptr = e->ptr;
    lease->kept = true;
    lease->hold = std::move(hold);
    return hipSuccess;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool log_enabled() {
    static const bool on = [] {
        const char* e = std::getenv("GQA_ATTN_LOG");
        return e && e[0] == '1';
    }();
    return on;
}

}  // namespace

extern "C" {

const char* gqa_attn_strerror(int status) {
    switch (status) {
        case GQA_OK: return "success";
        case GQA_ERR_INVALID_ARG: return "invalid argument";
        case GQA_ERR_UNSUPPORTED: return "unsupported head dimension or alignment";
        case GQA_ERR_NOMEM: return "split-KV workspace allocation failed";
        case GQA_ERR_HIP: return "HIP runtime or launch error";
        case GQA_ERR_SCRATCH: return "split-KV workspace larger than the fixed no-allocation scratch buffer";
        default: return "unknown status";
    }
}

int gqa_attn_choose(int B, int Sq, int Sk, int Hq, int Hk, int d, int causal, int num_cus,
                    int* pack_gqa, int* num_splits) {
    if (!pack_gqa || !num_splits) return GQA_ERR_INVALID_ARG;
    const gqa::Shape s{B, Sq, Sk, Hq, Hk, d, causal ? 1 : 0};
    const int st = gqa::check_sizes(s, 1.0f, -1, 0);
    if (st != GQA_OK) return st;
    if (num_cus <= 0) num_cus = device_cus(current_device());
    gqa::choose(s, num_cus, pack_gqa, num_splits);
    return GQA_OK;
}

int gqa_attn_plan(int B, int Sq, int Sk, int Hq, int Hk, int d, int causal, int pack_gqa,
                  int num_splits, int num_cus, gqa_attn_plan_t* plan) {
    if (!plan) return GQA_ERR_INVALID_ARG;
    const gqa::Shape s{B, Sq, Sk, Hq, Hk, d, causal ? 1 : 0};
    int st = gqa::check_sizes(s, 1.0f, pack_gqa, num_splits);
    if (st != GQA_OK) return st;
    if (num_cus <= 0) num_cus = device_cus(current_device());  // 0 without a device: make_plan assumes 256
    gqa::Plan p;
    st = gqa::make_plan(s, pack_gqa, num_splits, num_cus, &p);
    if (st != GQA_OK) return st;
    plan->pack_gqa = p.pack;
    plan->num_splits = p.ns;
    plan->block_m = p.block_m;
    plan->block_n = p.block_n;
    plan->row_tiles = p.row_tiles;
    plan->key_tiles = p.key_tiles;
    plan->grid = p.grid;
    plan->combine_grid = p.combine_grid;
    plan->workspace_bytes = p.workspace_bytes;
    plan->threads = p.threads;
    return GQA_OK;
}

}  // extern "C"

namespace {

// One forward call: contiguous K/V ([B, Sk, Hk, d]) or a paged pool.
struct Call {
    const void *q, *k, *v;
    void* out;
    float* lse;
    gqa::Shape s;  // for paged calls, Sk = the table's capacity max_pages * page_size
    float scale;
    int pack_gqa, num_splits;
    bool paged;
    const int* block_table;
    const int* seqlens_k;
    int page_size, max_pages, num_pages;
    hipStream_t stream;
    bool kv8 = false;       // fp8 e4m3 K/V with per-tensor factors
    float k_scale = 1.f, v_scale = 1.f;
    bool qk8 = false;       // fp8 e4m3 Q and K with per-tensor factors (q_scale, k_scale), bf16 V
    float q_scale = 1.f;
    bool varlen = false;    // packed sequences (s.Sq, s.Sk = max_seqlen_q, max_seqlen_k)
    const int* cu_q = nullptr;
    const int* cu_k = nullptr;
    int total_q = 0, total_k = 0;
    bool noalloc = false;   // split workspace from the fixed device scratch array, no allocation
};

int run(const Call& c) {
    const gqa::Shape& s = c.s;
    const int d = s.d;
    const int dev = current_device();
    if (dev < 0) return GQA_ERR_HIP;
    const int cus = device_cus(dev);  // cached per device
    gqa::Plan plan;
    int st = gqa::make_plan(s, c.pack_gqa, c.num_splits, cus, &plan);
    if (st != GQA_OK) return st;
    if (c.kv8 && !plan.decode) return GQA_ERR_UNSUPPORTED;  // fp8 K/V: decode kernel only

    gqa::FwdParams p{};
    p.q = (const uint16_t*)c.q;
    p.k = (const uint16_t*)c.k;
    p.v = (const uint16_t*)c.v;
    p.o = (uint16_t*)c.out;
    p.lse = c.lse;
    p.B = s.B;
    p.Sq = s.Sq;
    p.Sk = s.Sk;
    p.Hq = s.Hq;
    p.Hk = s.Hk;
    p.G = plan.G;
    p.Gp = plan.Gp;
    const gqa::FastDiv fd = gqa::make_fastdiv((uint32_t)plan.Gp);
    p.gmul = fd.mul;
    p.gshift = fd.shift;
    p.R = (int)plan.R;
    p.row_tiles = plan.row_tiles;
    p.units_per_b = plan.units_per_b;
    p.ns = plan.ns;
    p.grid = (int)plan.grid;
    p.pair_rows = plan.pair_rows;
    // softmax(scale * s) = softmax(|scale| * (sign(scale) * s)): a negative
    // scale negates Q (exact in bf16). scale == 0 gives every visible key
    // the score 0, which the kernel reproduces exactly by reading Q as 0.
    // A scale so small that |scale|*log2(e) is not a normal fp32 number
    // also gives every visible key exactly the same weight in fp32.
    // fp8 K/V: the scores are (scale * k_scale) * q.k8, the output v_scale * P.v8.
    // fp8 Q/K: the scores are (scale * q_scale * k_scale) * q8.k8 (the sign
    // bit of every e4m3 byte negates it).
    double score_scale = (double)c.scale;
    if (c.kv8) score_scale *= (double)c.k_scale;
    if (c.qk8) score_scale *= (double)c.q_scale * (double)c.k_scale;
    const double cd = std::fabs(score_scale) * 1.4426950408889634;
    const bool zero_scale = cd < 1.1754943508222875e-38;
    p.c = zero_scale ? 1.0f : (float)cd;
    p.qand = zero_scale ? 0u : 0xFFFFFFFFu;
    p.qsign = score_scale < 0.0 ? (c.qk8 ? 0x80808080u : 0x80008000u) : 0u;
    p.vscale = c.kv8 ? c.v_scale : 1.f;
    if (c.varlen) {
        p.cu_q = c.cu_q;
        p.cu_k = c.cu_k;
        p.total_q = c.total_q;
        p.total_k = c.total_k;
    }
    if (c.paged) {
        p.block_table = c.block_table;
        p.seqlens_k = c.seqlens_k;
        p.page_size = c.page_size;
        p.max_pages = c.max_pages;
        p.num_pages = c.num_pages;
        const gqa::FastDiv pd = gqa::make_fastdiv((uint32_t)c.page_size);
        p.pmul = pd.mul;
        p.pshift = pd.shift;
    }

    if (log_enabled())
        std::fprintf(stderr,
                     "[gqa_attn] B=%d Sq=%d Sk=%d Hq=%d Hk=%d d=%d causal=%d paged=%d kv8=%d -> pack=%d ns=%d "
                     "kernel=%s row_tiles=%d key_tiles=%d grid=%lld combine_grid=%lld ws=%lld\n",
                     s.B, s.Sq, s.Sk, s.Hq, s.Hk, d, s.causal, c.paged ? 1 : 0, c.kv8 ? 1 : 0, plan.pack, plan.ns,
                     plan.decode ? "decode" : (plan.pingpong ? "tiled8" : "tiled"), plan.row_tiles, plan.key_tiles, plan.grid,
                     plan.combine_grid, plan.workspace_bytes);

    auto launch = [&](bool split) {
        if (plan.pingpong) return gqa::launch_pingpong(p, d, s.causal != 0, c.paged, c.varlen, c.qk8, c.stream);  // unsplit only
        return plan.decode ? gqa::launch_decode(p, d, s.causal != 0, split, c.paged, c.kv8, c.varlen, c.stream)
                           : gqa::launch_attention(p, d, s.causal != 0, split, c.varlen, c.qk8, c.paged, c.stream);
    };
    // variable-length prefill whose sequences leave most of the grid empty runs
    // from a work list that a scheduling kernel builds on the device: the
    // (sequence, row tile) pairs that exist, heaviest first. The list holds at
    // most one partial row tile per sequence beyond the full ones the packed
    // tokens fill. The 8-wavefront kernel takes variable-length calls only so.
    const bool sched = plan.worklist != 0;
    if (plan.pingpong && c.varlen && !sched) return GQA_ERR_UNSUPPORTED;
    long long sched_cap = 0;
    size_t sched_bytes = 0;
    // causal calls on the 8-wavefront kernel list pairs of row tiles: ceil(R_b / 2)
    // entries per sequence, at most total_q * Gp / (2 * block_m) + B of them
    const bool sched_pairs = sched && plan.pingpong && s.causal;
    if (sched) {
        const long long per = sched_pairs ? 2LL * plan.block_m : plan.block_m;
        sched_cap = ((long long)c.total_q * plan.Gp + per - 1) / per + s.B;
        const long long grid = sched_cap * plan.units_per_b * plan.ns;
        if (sched_cap > INT_MAX / 4 || grid > INT_MAX) return GQA_ERR_INVALID_ARG;
        p.grid = (int)grid;
        sched_bytes = (((size_t)(1 + 2 * sched_cap) * 4) + 255) & ~(size_t)255;
    }
    if (plan.ns == 1 && !sched) {
        hipError_t e = launch(false);
        return e == hipSuccess ? GQA_OK : GQA_ERR_HIP;
    }

    void* ws = nullptr;
    WsLease lease;  // a kept buffer stays held until this call's kernels are enqueued
    const size_t split_bytes = plan.ns == 1 ? 0
                               : c.varlen ? (size_t)plan.ns * (size_t)c.total_q * s.Hq * ((size_t)d * 4 + 8)
                                          : (size_t)plan.workspace_bytes;
    const size_t ws_bytes = sched_bytes + split_bytes;
    if (c.noalloc) {
        // every partial the combine reads is written by this call's attention
        // kernel (empty splits write O_s = 0, LSE_s = -inf), so nothing is cleared
        if (ws_bytes > (size_t)gqa::kScratchBytes) return GQA_ERR_SCRATCH;
        if (gqa::scratch_address(dev, &ws) != hipSuccess || !ws) return GQA_ERR_HIP;
    } else {
        if (ws_acquire(ws_bytes, dev, c.stream, &lease) != hipSuccess || !lease.ptr) {
            (void)hipGetLastError();
            return GQA_ERR_NOMEM;
        }
        ws = lease.ptr;
    }
    const int64_t rows = c.varlen ? (int64_t)c.total_q * s.Hq : (int64_t)s.B * s.Sq * s.Hq;
    hipError_t e = hipSuccess;
    if (sched) {
        gqa::SchedParams sp{};
        sp.cu_q = c.cu_q;
        sp.cu_k = c.cu_k;
        sp.worklist = (int*)ws;
        sp.B = s.B;
        sp.total_q = c.total_q;
        sp.total_k = c.total_k;
        sp.max_sq = s.Sq;
        sp.Gp = plan.Gp;
        sp.gmul = fd.mul;
        sp.gshift = fd.shift;
        sp.block_m = plan.block_m;
        sp.causal = s.causal;
        sp.pair = sched_pairs ? 1 : 0;
        sp.cap = (int)sched_cap;
        p.worklist = (const int*)ws;
        e = gqa::launch_schedule(sp, c.stream);
    }
    float* parts = (float*)((char*)ws + sched_bytes);
    p.opart = parts;
    p.lpart = parts + (int64_t)plan.ns * rows * d;
    p.wpart = p.lpart + (int64_t)plan.ns * rows;
    if (e == hipSuccess) e = launch(plan.ns > 1);
    if (e == hipSuccess && plan.ns > 1) {
        gqa::CombineParams cp{};
        cp.opart = p.opart;
        cp.lpart = p.lpart;
        cp.wpart = p.wpart;
        cp.o = (uint16_t*)c.out;
        cp.lse = c.lse;
        cp.rows = rows;
        cp.ns = plan.ns;
        cp.Sq = c.varlen ? c.total_q : s.Sq;  // varlen: lse [Hq, total_q] = one batch of total_q tokens
        cp.Hq = s.Hq;
        if (c.varlen) {
            cp.cu_q = c.cu_q;
            cp.B = s.B;
            cp.total_q = c.total_q;
            cp.max_sq = s.Sq;
        }
        // variable-length calls: the workspace has total_q * Hq rows (the plan counts B * max_seqlen_q * Hq)
        const long long cgrid = !c.varlen ? plan.combine_grid
                                : plan.ns >= gqa::kCombineWideSplits ? (long long)rows
                                                                     : ((long long)rows + gqa::combine_rows_per_block(d) - 1) /
                                                                           gqa::combine_rows_per_block(d);
        if (cgrid > INT_MAX) e = hipErrorInvalidValue;
        else e = gqa::launch_combine(cp, d, cgrid, c.stream);
    }
    const hipError_t ef = (c.noalloc || lease.kept) ? hipSuccess : hipFreeAsync(ws, c.stream);
    if (e != hipSuccess || ef != hipSuccess) return GQA_ERR_HIP;
    return GQA_OK;
}

bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

}  // namespace

extern "C" {

int gqa_attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Sq,
                 int Sk, int Hq, int Hk, int d, int causal, float scale, int pack_gqa, int num_splits,
                 hipStream_t stream) {
    try {
        const gqa::Shape s{B, Sq, Sk, Hq, Hk, d, causal ? 1 : 0};
        int st = gqa::check_sizes(s, scale, pack_gqa, num_splits);
        if (st != GQA_OK) return st;
        if ((long long)B * Sq == 0) return GQA_OK;
        if (!q || !k || !v || !out) return GQA_ERR_INVALID_ARG;
        if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return GQA_ERR_UNSUPPORTED;
        Call c{q, k, v, out, lse, s, scale, pack_gqa, num_splits, false, nullptr, nullptr, 0, 0, 0, stream};
        return run(c);
    } catch (...) {
        return GQA_ERR_HIP;
    }
}

int gqa_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Sq,
                         int Sk, int Hq, int Hk, int d, int causal, float scale, int pack_gqa, int num_splits,
                         hipStream_t stream) {
    try {
        const gqa::Shape s{B, Sq, Sk, Hq, Hk, d, causal ? 1 : 0};
        int st = gqa::check_sizes(s, scale, pack_gqa, num_splits);
        if (st != GQA_OK) return st;
        if ((long long)B * Sq == 0) return GQA_OK;
        if (!q || !k || !v || !out) return GQA_ERR_INVALID_ARG;
        if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return GQA_ERR_UNSUPPORTED;
        // the first call on a device looks up that device's copy of the scratch array
        void* scratch = nullptr;
        if (gqa::scratch_address(current_device(), &scratch) != hipSuccess || !scratch) return GQA_ERR_HIP;
        Call c{q, k, v, out, lse, s, scale, pack_gqa, num_splits, false, nullptr, nullptr, 0, 0, 0, stream};
        c.noalloc = true;
        return run(c);
    } catch (...) {
        return GQA_ERR_HIP;
    }
}

int gqa_attn_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse, const void* dout,
                 void* dq, void* dk, void* dv, int B, int Sq, int Sk, int Hq, int Hk, int d, int causal, float scale,
                 hipStream_t stream) {
    try {
        const gqa::Shape s{B, Sq, Sk, Hq, Hk, d, causal ? 1 : 0};
        int st = gqa::check_sizes(s, scale, -1, 0);
        if (st != GQA_OK) return st;
        if ((long long)B * Sq == 0 && (long long)B * Sk == 0) return GQA_OK;
        // without query rows only dK = dV = 0 is written (from k and v's shapes): the
        // query-side pointers may be null then
        const bool has_rows = (long long)B * Sq > 0;
        if (!k || !v || !dk || !dv || (has_rows && (!q || !out || !lse || !dout || !dq))) return GQA_ERR_INVALID_ARG;
        if (!aligned16(k) || !aligned16(v) || !aligned16(dk) || !aligned16(dv) ||
            (has_rows && (!aligned16(q) || !aligned16(out) || !aligned16(dout) || !aligned16(dq) || !aligned4(lse))))
            return GQA_ERR_UNSUPPORTED;
        // per-batch byte offsets of the query tiles are 32-bit
        if ((long long)Sq * Hq * d * 2 > 0x7FFFFFFFLL || (long long)Hq * Sq * 4 > 0x7FFFFFFFLL) return GQA_ERR_INVALID_ARG;
        const int G = Hq / Hk;
        if ((long long)Sq * G > INT_MAX / 2) return GQA_ERR_INVALID_ARG;
        gqa::BwdParams p{};
        p.q = (const uint16_t*)q;
        p.k = (const uint16_t*)k;
        p.v = (const uint16_t*)v;
        p.o = (const uint16_t*)out;
        p.dout = (const uint16_t*)dout;
        p.lse = lse;
        p.dq = (uint16_t*)dq;
        p.dk = (uint16_t*)dk;
        p.dv = (uint16_t*)dv;
        p.B = B;
        p.Sq = Sq;
        p.Sk = Sk;
        p.Hq = Hq;
        p.Hk = Hk;
        p.G = G;
        const gqa::FastDiv fd = gqa::make_fastdiv((uint32_t)G);
        p.gmul = fd.mul;
        p.gshift = fd.shift;
        p.R = Sq * G;
        p.row_tiles = (p.R + gqa::kBlockM - 1) / gqa::kBlockM;
        p.key_blocks = (Sk + gqa::kBwdKeys - 1) / gqa::kBwdKeys;
        const long long gdq = (long long)B * Hk * p.row_tiles, gkv = (long long)B * Hk * p.key_blocks;
        if (gdq > INT_MAX || gkv > INT_MAX) return GQA_ERR_INVALID_ARG;
        p.grid_dq = (int)gdq;
        p.grid_dkdv = (int)gkv;
        p.c = (float)((double)scale * 1.4426950408889634);
        p.scale = scale;
        if (current_device() < 0) return GQA_ERR_HIP;
        const int dev = current_device();
        void* ws = nullptr;
        const size_t rows = (size_t)B * Hq * (size_t)(Sq > 0 ? Sq : 1);
        const size_t ws_bytes = 2 * rows * 4;  // D, then -LSE*log2(e)
        WsLease lease;  // a kept buffer stays held until the kernels are enqueued
        if (ws_acquire(ws_bytes, dev, stream, &lease) != hipSuccess || !lease.ptr) {
            (void)hipGetLastError();
            return GQA_ERR_NOMEM;
        }
        ws = lease.ptr;
        p.drow = (float*)ws;
        p.nlse2 = (float*)ws + rows;
        const hipError_t e = gqa::launch_backward(p, d, causal != 0, stream);
        const hipError_t ef = lease.kept ? hipSuccess : hipFreeAsync(ws, stream);
        if (e != hipSuccess || ef != hipSuccess) return GQA_ERR_HIP;
        return GQA_OK;
    } catch (...) {
        return GQA_ERR_HIP;
    }
}

int gqa_attn_fwd_varlen(const void* q, const void* k, const void* v, void* out, float* lse,
                        const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int max_seqlen_q,
                        int max_seqlen_k, int total_q, int total_k, int Hq, int Hk, int d, int causal,
                        float scale, int pack_gqa, int num_splits, hipStream_t stream) {
    try {
        if (total_q < 0 || total_k < 0) return GQA_ERR_INVALID_ARG;
        gqa::Shape s{B, max_seqlen_q, max_seqlen_k, Hq, Hk, d, causal ? 1 : 0, 2, 2, 1};
        s.total_q = total_q;
        int st = gqa::check_sizes(s, scale, pack_gqa, num_splits);
        if (st != GQA_OK) return st;
        if ((long long)B * max_seqlen_q == 0 || total_q == 0) return GQA_OK;
        if (!q || !k || !v || !out || !cu_seqlens_q || !cu_seqlens_k) return GQA_ERR_INVALID_ARG;
        if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned4(cu_seqlens_q) ||
            !aligned4(cu_seqlens_k))
            return GQA_ERR_UNSUPPORTED;
        Call c{q, k, v, out, lse, s, scale, pack_gqa, num_splits, false, nullptr, nullptr, 0, 0, 0, stream};
        c.varlen = true;
        c.cu_q = cu_seqlens_q;
        c.cu_k = cu_seqlens_k;
        c.total_q = total_q;
        c.total_k = total_k;
        return run(c);
    } catch (...) {
        return GQA_ERR_HIP;
    }
}

static int fwd_paged(const void* q, const void* k_cache, const void* v_cache, const int* block_table,
                     const int* seqlens_k, void* out, float* lse, int B, int Sq, int Hq, int Hk, int d,
                     int num_pages, int page_size, int max_pages, int causal, float scale, int pack_gqa,
                     int num_splits, hipStream_t stream, bool kv8, float k_scale, float v_scale) {
    try {
        if (page_size <= 0 || max_pages <= 0 || num_pages <= 0) return GQA_ERR_INVALID_ARG;
        if ((long long)max_pages * page_size > INT_MAX / 2) return GQA_ERR_INVALID_ARG;
        if (kv8 && (!std::isfinite(k_scale) || !std::isfinite(v_scale))) return GQA_ERR_INVALID_ARG;
        gqa::Shape s{B, Sq, max_pages * page_size, Hq, Hk, d, causal ? 1 : 0, kv8 ? 1 : 2};
        s.paged = 1;
        int st = gqa::check_sizes(s, scale, pack_gqa, num_splits);
        if (st != GQA_OK) return st;
        if (page_size % 16 != 0) return GQA_ERR_UNSUPPORTED;
        if ((long long)page_size * Hk * d * (kv8 ? 1 : 2) > INT_MAX) return GQA_ERR_INVALID_ARG;  // 32-bit in-page offsets
        if (kv8) {  // fp8 pools: decode-shaped calls only (the pack decision does not depend on the CU count)
            gqa::Plan probe;
            st = gqa::make_plan(s, pack_gqa, num_splits, 256, &probe);
            if (st != GQA_OK) return st;
            if (!probe.decode) return GQA_ERR_UNSUPPORTED;
        }
        if ((long long)B * Sq == 0) return GQA_OK;
        if (!q || !k_cache || !v_cache || !block_table || !seqlens_k || !out) return GQA_ERR_INVALID_ARG;
        if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
            !aligned4(block_table) || !aligned4(seqlens_k))
            return GQA_ERR_UNSUPPORTED;
        Call c{q, k_cache, v_cache, out, lse, s, scale, pack_gqa, num_splits, true, block_table, seqlens_k,
               page_size, max_pages, num_pages, stream, kv8, k_scale, v_scale};
        return run(c);
    } catch (...) {
        return GQA_ERR_HIP;
    }
}

int gqa_attn_fwd_paged(const void* q, const void* k_cache, const void* v_cache, const int* block_table,
                       const int* seqlens_k, void* out, float* lse, int B, int Sq, int Hq, int Hk, int d,
                       int num_pages, int page_size, int max_pages, int causal, float scale, int pack_gqa,
                       int num_splits, hipStream_t stream) {
    return fwd_paged(q, k_cache, v_cache, block_table, seqlens_k, out, lse, B, Sq, Hq, Hk, d, num_pages, page_size,
                     max_pages, causal, scale, pack_gqa, num_splits, stream, false, 1.f, 1.f);
}

int gqa_attn_fwd_kv8(const void* q, const void* k, const void* v, float k_scale, float v_scale, void* out,
                     float* lse, int B, int Sq, int Sk, int Hq, int Hk, int d, int causal, float scale,
                     int pack_gqa, int num_splits, hipStream_t stream) {
    try {
        if (!std::isfinite(k_scale) || !std::isfinite(v_scale)) return GQA_ERR_INVALID_ARG;
        const gqa::Shape s{B, Sq, Sk, Hq, Hk, d, causal ? 1 : 0, 1};
        int st = gqa::check_sizes(s, scale, pack_gqa, num_splits);
        if (st != GQA_OK) return st;
        {
            gqa::Plan probe;
            st = gqa::make_plan(s, pack_gqa, num_splits, 256, &probe);
            if (st != GQA_OK) return st;
            if (!probe.decode) return GQA_ERR_UNSUPPORTED;
        }
        if ((long long)B * Sq == 0) return GQA_OK;
        if (!q || !k || !v || !out) return GQA_ERR_INVALID_ARG;
        if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return GQA_ERR_UNSUPPORTED;
        Call c{q, k, v, out, lse, s, scale, pack_gqa, num_splits, false, nullptr, nullptr, 0, 0, 0, stream,
               true, k_scale, v_scale};
        return run(c);
    } catch (...) {
        return GQA_ERR_HIP;
    }
}

int gqa_attn_fwd_qk8(const void* q, const void* k, const void* v, float q_scale, float k_scale, void* out,
                     float* lse, int B, int Sq, int Sk, int Hq, int Hk, int d, int causal, float scale,
                     int pack_gqa, int num_splits, hipStream_t stream) {
    try {
        if (!std::isfinite(q_scale) || !std::isfinite(k_scale)) return GQA_ERR_INVALID_ARG;
        gqa::Shape s{B, Sq, Sk, Hq, Hk, d, causal ? 1 : 0};
        s.q_bytes = 1;
        int st = gqa::check_sizes(s, scale, pack_gqa, num_splits);
        if (st != GQA_OK) return st;
        if ((long long)B * Sq == 0) return GQA_OK;
        if (!q || !k || !v || !out) return GQA_ERR_INVALID_ARG;
        if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return GQA_ERR_UNSUPPORTED;
        Call c{q, k, v, out, lse, s, scale, pack_gqa, num_splits, false, nullptr, nullptr, 0, 0, 0, stream};
        c.qk8 = true;
        c.q_scale = q_scale;
        c.k_scale = k_scale;
        return run(c);
    } catch (...) {
        return GQA_ERR_HIP;
    }
}

int gqa_attn_fwd_paged_kv8(const void* q, const void* k_cache, const void* v_cache, float k_scale, float v_scale,
                           const int* block_table, const int* seqlens_k, void* out, float* lse, int B, int Sq,
                           int Hq, int Hk, int d, int num_pages, int page_size, int max_pages, int causal,
                           float scale, int pack_gqa, int num_splits, hipStream_t stream) {
    return fwd_paged(q, k_cache, v_cache, block_table, seqlens_k, out, lse, B, Sq, Hq, Hk, d, num_pages, page_size,
                     max_pages, causal, scale, pack_gqa, num_splits, stream, true, k_scale, v_scale);
}

}  // extern "C"
