// fa_varlen.hip -- work list of a packed variable-length (TND) prefill.
//
// The packed layout (FlashAttn developer guide 1.3) removes the padding of a
// ragged batch, which leaves its query tiles (128 or 256 rows, as the prefill
// kernel that runs takes them) with very different
// costs: a tile of a long sequence visits many more KV tiles than one of a
// short sequence, and under a causal mask the last tiles of a sequence cost
// the most.  The developer guide balances such work with a cost model over
// blocks (section 4, SectionStreamK: cost grows with the rows and the KV blocks
// of a block) computed into metadata before the kernel runs.  Here the same
// job is one workgroup on the device, so the offsets never travel to the host:
// it enumerates every (sequence, q tile) item, prices it as the number of
// 64-key KV tiles the prefill kernel will visit plus a fixed two-tile overhead,
// and writes the items heaviest first (a counting sort over the cost).  The
// hardware dispatcher hands workgroups out in that order as CUs free up, so
// this is longest-processing-time-first scheduling; the prefill kernel deals
// consecutive items to different XCDs.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

constexpr int kSchedThreads = 1024;
constexpr int kCostBins = 4096;

__device__ __forceinline__ int tile_cost(const VarlenScheduleArgs& a, const SeqGeom& g, int64_t qt) {
    const int64_t i0 = qt * a.rows;
    if (i0 >= g.q_used) return 1;  // only writes the initial values
    int64_t kv_end = g.kv_len;
    int64_t jt0 = 0;
    if (a.mask_mode == 1 && kv_end > i0 + a.rows) kv_end = i0 + a.rows;
    if (a.mask_mode == 4) {
        const int64_t i_last = (i0 + a.rows < g.q_used ? i0 + a.rows : g.q_used) - 1;
        if (kv_end > i_last + a.win_right + 1) kv_end = i_last + a.win_right + 1;
        const int64_t lo = i0 - a.win_left;
        if (lo > 0) jt0 = lo / 64;
    }
    int64_t n = (kv_end + 63) / 64 - jt0;
    if (n < 0) n = 0;
    const int64_t c = n + 2;
    return (int)(c < kCostBins ? c : kCostBins - 1);
}

__global__ __launch_bounds__(kSchedThreads) void varlen_schedule_kernel(VarlenScheduleArgs a) {
    // s_start[s] = first item of sequence s (sequence `batch` = rows past the last one).
    __shared__ int32_t s_start[kVarlenMaxBatch + 3];
    __shared__ int32_t s_hist[kCostBins];
    __shared__ int32_t s_part[kSchedThreads];
    const int t = threadIdx.x;
    const int nseq = a.batch + 1;

    for (int s = t; s < nseq; s += kSchedThreads) {
        const SeqGeom g = seq_geometry(a.cu_q, a.cu_kv, a.used_q, a.lens, s, a.batch, a.q_total, a.kv_total);
        s_start[s + 1] = (int32_t)((g.q_full + a.rows - 1) / a.rows);
    }
    if (t == 0) s_start[0] = 0;
    for (int i = t; i < kCostBins; i += kSchedThreads) s_hist[i] = 0;
    __syncthreads();

    // Inclusive scan of the tile counts: per-thread segments, then a scan of
    // the segment sums.
    const int seg = (nseq + kSchedThreads - 1) / kSchedThreads;
    const int lo = 1 + t * seg;
    const int hi = (lo + seg < nseq + 1) ? lo + seg : nseq + 1;
    int sum = 0;
    for (int i = lo; i < hi; ++i) sum += s_start[i];
    s_part[t] = sum;
    __syncthreads();
    for (int off = 1; off < kSchedThreads; off <<= 1) {
        const int v = (t >= off) ? s_part[t - off] : 0;
        __syncthreads();
        s_part[t] += v;
        __syncthreads();
    }
    int run = (t > 0) ? s_part[t - 1] : 0;
    for (int i = lo; i < hi; ++i) {
        run += s_start[i];
        s_start[i] = run;
    }
    __syncthreads();
    int total = s_start[nseq];
    if (total > a.capacity) total = a.capacity;  // the host sizes the list; never write past it

    // Item -> (sequence, q tile): the last sequence whose first item is <= it.
    auto locate = [&](int it, int* sq, int* qt) __attribute__((always_inline)) {
        int l = 0, h = nseq;  // s_start[l] <= it < s_start[h]
        while (h - l > 1) {
            const int m = (l + h) >> 1;
            if (s_start[m] <= it) l = m;
            else h = m;
        }
        *sq = l;
        *qt = it - s_start[l];
    };

    for (int it = t; it < total; it += kSchedThreads) {
        int sq, qt;
        locate(it, &sq, &qt);
        const SeqGeom g = seq_geometry(a.cu_q, a.cu_kv, a.used_q, a.lens, sq, a.batch, a.q_total, a.kv_total);
        atomicAdd(&s_hist[tile_cost(a, g, qt)], 1);
    }
    __syncthreads();

    // Exclusive scan in descending cost order: bin c starts after every item
    // that costs more.  Thread t owns the four bins counted from the top.
    constexpr int BPT = kCostBins / kSchedThreads;
    int cnt[BPT];
    int local = 0;
#pragma unroll
    for (int k = 0; k < BPT; ++k) {
        cnt[k] = s_hist[kCostBins - 1 - (t * BPT + k)];
        local += cnt[k];
    }
    s_part[t] = local;
    __syncthreads();
    for (int off = 1; off < kSchedThreads; off <<= 1) {
        const int v = (t >= off) ? s_part[t - off] : 0;
        __syncthreads();
        s_part[t] += v;
        __syncthreads();
    }
    int base = (t > 0) ? s_part[t - 1] : 0;
#pragma unroll
    for (int k = 0; k < BPT; ++k) {
        s_hist[kCostBins - 1 - (t * BPT + k)] = base;
        base += cnt[k];
    }
    __syncthreads();

    for (int it = t; it < total; it += kSchedThreads) {
        int sq, qt;
        locate(it, &sq, &qt);
        const SeqGeom g = seq_geometry(a.cu_q, a.cu_kv, a.used_q, a.lens, sq, a.batch, a.q_total, a.kv_total);
        const int pos = atomicAdd(&s_hist[tile_cost(a, g, qt)], 1);
        a.work[2 * pos] = sq;
        a.work[2 * pos + 1] = qt;
    }
    for (int i = total + t; i < a.capacity; i += kSchedThreads) {
        a.work[2 * i] = -1;
        a.work[2 * i + 1] = -1;
    }
}

hipError_t launch_varlen_schedule(const VarlenScheduleArgs& a, hipStream_t stream) {
    if (a.batch < 0 || a.batch > kVarlenMaxBatch || a.capacity <= 0 || (a.rows != 128 && a.rows != 256))
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(varlen_schedule_kernel, dim3(1), dim3(kSchedThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace fa
