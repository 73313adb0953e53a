// fa_masksum.hip -- per-tile summary of a boolean mask tensor for the prefill.
//
// A mask given as a tensor hides its structure from the prefill kernel: under
// a causal pattern half of the KV tiles of a query tile hold no visible key,
// and most of the rest hold no masked one.  For the window mode the
// FlashAttn developer guide (1.5) has the kernel skip the tiles with no valid
// key from the band's bounds; for a tensor mask the same facts are read from
// the tensor once, before the prefill runs.  One workgroup of 16 waves covers
// one (mask slice, 128-row query tile, 16 KV tiles of 64 keys): each wave
// reads eight rows of the slab, 16 bytes per lane with all eight loads in
// flight, and records whether it saw a zero byte (a visible key) and a
// non-zero byte (a masked key); a ballot per wave and an OR over the waves
// give two bits per KV tile.
//
// The prefill then visits only the KV tiles between the first and the last
// tile with a visible key, issues no loads for tiles in between that have
// none, and skips both the mask load and the element tests of tiles that mask
// nothing.  Every skipped tile is one the prefill would have found fully
// masked (or mask-free) itself, so its results do not change.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

constexpr int kSumThreads = 1024;
constexpr int kSumWaves = kSumThreads / 64;

__global__ __launch_bounds__(kSumThreads) void mask_summary_kernel(MaskSummaryArgs a) {
    constexpr int RPW = kMaskRowsPerTile / kSumWaves;  // rows per wave
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t id = blockIdx.x;
    if (id >= a.blocks) return;
    const int64_t w = id % a.words;
    const int64_t rest = id / a.words;
    const int64_t qt = rest % a.q_tiles;
    const int64_t sl = rest / a.q_tiles;
    const int64_t sb = sl / a.slices_n;
    const int64_t sn = sl % a.slices_n;

    const int64_t row0 = qt * kMaskRowsPerTile;
    int64_t rows = a.q_seq - row0;
    rows = rows > kMaskRowsPerTile ? kMaskRowsPerTile : rows;
    // Lane covers keys [key, key + 16) of the word's 1024; kv_seq is a
    // multiple of 16, so a chunk is either wholly inside the row or past it.
    const int64_t key = w * (kMaskTilesPerWord * kMaskKeysPerTile) + 16 * lane;
    const uint8_t* base = a.mask + sb * a.mask_stride[0] + sn * a.mask_stride[1] + row0 * a.mask_stride[2] + key;
    // zero_bits collects the high bit of every zero byte seen (a visible
    // key), any_bits every bit of every byte (a masked key).
    uint32_t zero_bits = 0u, any_bits = 0u;
    if (key < a.kv_seq) {
        u32x4 x[RPW];
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            // Rows past the query length re-read the last row (rows >= 1),
            // which leaves both flags unchanged and keeps the loads unbranched.
            int64_t r = (int64_t)wave * RPW + i;
            r = r < rows ? r : rows - 1;
            x[i] = ld128(base + r * a.mask_stride[2]);
        }
#pragma unroll
        for (int i = 0; i < RPW; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                zero_bits |= (x[i][e] - 0x01010101u) & ~x[i][e] & 0x80808080u;
                any_bits |= x[i][e];
            }
    }
    const bool vis = zero_bits != 0u, msk = any_bits != 0u;
    // Lanes 4t .. 4t+3 hold the 64 keys of KV tile t of the word.
    __shared__ uint64_t s_vis[kSumWaves], s_msk[kSumWaves];
    const uint64_t bv = __ballot(vis);
    const uint64_t bm = __ballot(msk);
    if (lane == 0) {
        s_vis[wave] = bv;
        s_msk[wave] = bm;
    }
    __syncthreads();
    if (tid == 0) {
        uint64_t v = 0, m = 0;
#pragma unroll
        for (int i = 0; i < kSumWaves; ++i) {
            v |= s_vis[i];
            m |= s_msk[i];
        }
        uint32_t word = 0;
#pragma unroll
        for (int t = 0; t < kMaskTilesPerWord; ++t) {
            const uint32_t c = (((v >> (4 * t)) & 0xfu) ? 1u : 0u) | (((m >> (4 * t)) & 0xfu) ? 2u : 0u);
            word |= c << (2 * t);
        }
        a.out[id] = word;
    }
}

hipError_t launch_mask_summary(const MaskSummaryArgs& a, hipStream_t stream) {
    if (a.blocks <= 0 || a.blocks > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(mask_summary_kernel, dim3((unsigned)a.blocks), dim3(kSumThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace fa
