// Work list of a variable-length prefill call.
//
// For packed sequences of very different lengths, the tiled kernels' plain
// grid would hold an item for every row tile of the longest sequence in every
// sequence, most of which exit at once, and would start the items in an
// order unrelated to their cost. This kernel lists the (sequence, row tile)
// pairs that exist, ordered by the key tiles each one reads (heaviest first,
// so the long causal tiles of all sequences start first and the short ones
// fill the tail): a counting sort over the cost with one LDS histogram.
//
// One workgroup of 1024 threads. Sequences are taken 1024 at a time: thread
// t clamps sequence t's extent exactly as the attention kernels do, an
// exclusive scan of the row-tile counts numbers the chunk's pairs, and the
// threads then take the pairs in turn (a binary search of the scan gives the
// sequence of a pair). The first pass counts the pairs per cost bin; a scan
// of the bins from the heaviest turns the counts into start slots; the second
// pass takes a slot per pair and writes it. Pairs of equal cost land in any
// order: the results do not depend on the order.
//
// Pair mode (causal calls on the 8-wavefront kernel): an entry (b, pr) stands
// for row tiles R_b-1-pr and pr of sequence b, which one workgroup runs one
// after the other (the middle tile of an odd count alone); its cost is the key
// tiles of both, and sequence b has ceil(R_b / 2) entries.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "kernels.h"

namespace gqa {

namespace {

constexpr int kWaves = kSchedThreads / 64;

// Exclusive prefix sum of v over the workgroup's threads in thread order;
// *total receives the sum of all. wsum: kWaves ints of LDS. Every thread
// must call it (it holds two barriers).
__device__ __forceinline__ int block_exclusive_scan(int v, int* wsum, int* total) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    if (w == 0) {
        int t = lane < kWaves ? wsum[lane] : 0;
#pragma unroll
        for (int off = 1; off < kWaves; off <<= 1) {
            const int y = __shfl_up(t, off, 64);
            if (lane >= off) t += y;
        }
        if (lane < kWaves) wsum[lane] = t;
    }
    __syncthreads();
    *total = wsum[kWaves - 1];
    return x - v + (w > 0 ? wsum[w - 1] : 0);
}

}  // namespace

__global__ __launch_bounds__(kSchedThreads) void varlen_schedule_kernel(const SchedParams sp) {
    static_assert(kSchedThreads == kSchedBins && kSchedThreads == 1024, "one bin per thread, 16 wavefronts");
    __shared__ int bins[kSchedBins];          // pairs per cost bin, then each bin's next free slot
    __shared__ int seq_off[kSchedThreads + 1];  // the chunk's first pair of each sequence; [1024] = its pairs
    __shared__ int seq_q[kSchedThreads], seq_k[kSchedThreads];  // the chunk's clamped query and key counts
    __shared__ int wsum[kWaves];
    const int tid = threadIdx.x;
    bins[tid] = 0;
    __syncthreads();

    // the key tiles that row tile rt of a sequence reads (the attention
    // kernels' count)
    auto tiles = [&](int Sq, int Sk, int rt) {
        int kv_end = Sk;
        if (sp.causal) {
            const int r_last = min((rt + 1) * sp.block_m, Sq * sp.Gp) - 1;
            const int i_max = (int)fdiv((uint32_t)r_last, sp.gmul, sp.gshift);
            kv_end = min(Sk, i_max + (Sk - Sq) + 1);
        }
        return kv_end > 0 ? (kv_end + kBlockN - 1) / kBlockN : 0;
    };
    // the cost of entry e of a sequence (row tile e; pair mode: row tiles
    // R-1-e and e), as a bin
    auto cost_bin = [&](int Sq, int Sk, int e) {
        int T;
        if (sp.pair) {
            const int R = (Sq * sp.Gp + sp.block_m - 1) / sp.block_m;
            const int rt1 = R - 1 - e;
            T = tiles(Sq, Sk, rt1) + (e < rt1 ? tiles(Sq, Sk, e) : 0);
        } else {
            T = tiles(Sq, Sk, e);
        }
        return min(T, kSchedBins - 1);
    };
    // sequences c0 .. c0+1023 into seq_q, seq_k, seq_off; returns the chunk's pairs
    auto load_chunk = [&](int c0) {
        const int b = c0 + tid;
        int Sq = 0, Sk = 0, nt = 0;
        if (b < sp.B) {
            const int a0 = sp.cu_q[b], a1 = sp.cu_q[b + 1], k0r = sp.cu_k[b], k1r = sp.cu_k[b + 1];
            const int q0 = min(max(a0, 0), sp.total_q);
            const int q1 = min(max(a1, q0), sp.total_q);
            const int k0 = min(max(k0r, 0), sp.total_k);
            const int k1 = min(max(k1r, k0), sp.total_k);
            Sq = min(q1 - q0, sp.max_sq);
            Sk = k1 - k0;
            nt = (Sq * sp.Gp + sp.block_m - 1) / sp.block_m;
            if (sp.pair) nt = (nt + 1) >> 1;  // entries of the sequence
        }
        seq_q[tid] = Sq;
        seq_k[tid] = Sk;
        int total;
        seq_off[tid] = block_exclusive_scan(nt, wsum, &total);
        if (tid == 0) seq_off[kSchedThreads] = total;
        __syncthreads();
        return total;
    };
    // the chunk's sequence (index in the chunk) that holds pair p
    auto seq_of = [&](int p) {
        int lo = 0, hi = kSchedThreads;  // seq_off[lo] <= p < seq_off[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (seq_off[mid] <= p) lo = mid; else hi = mid;
        }
        return lo;
    };

    // pass 1: pairs per cost bin
    int pairs = 0;
    for (int c0 = 0; c0 < sp.B; c0 += kSchedThreads) {
        pairs = load_chunk(c0);
        for (int p = tid; p < pairs; p += kSchedThreads) {
            const int j = seq_of(p);
            atomicAdd(&bins[cost_bin(seq_q[j], seq_k[j], p - seq_off[j])], 1);
        }
        __syncthreads();
    }
    // start slot of each bin, heaviest bin first: thread t scans bin 1023-t
    {
        const int cnt = bins[kSchedBins - 1 - tid];
        int total;
        const int start = block_exclusive_scan(cnt, wsum, &total);
        bins[kSchedBins - 1 - tid] = start;
        if (tid == 0) sp.worklist[0] = min(total, sp.cap);
        __syncthreads();
    }
    // pass 2: a slot per pair (one chunk of at most 1024 sequences is still in LDS)
    for (int c0 = 0; c0 < sp.B; c0 += kSchedThreads) {
        if (sp.B > kSchedThreads) pairs = load_chunk(c0);
        for (int p = tid; p < pairs; p += kSchedThreads) {
            const int j = seq_of(p);
            const int rt = p - seq_off[j];
            const int slot = atomicAdd(&bins[cost_bin(seq_q[j], seq_k[j], rt)], 1);
            if (slot < sp.cap) {
                sp.worklist[1 + 2 * slot] = c0 + j;
                sp.worklist[2 + 2 * slot] = rt;
            }
        }
        __syncthreads();
    }
}

hipError_t launch_schedule(const SchedParams& sp, hipStream_t stream) {
    hipLaunchKernelGGL(varlen_schedule_kernel, dim3(1), dim3(kSchedThreads), 0, stream, sp);
    return hipGetLastError();
}

}  // namespace gqa
