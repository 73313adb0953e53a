// fa_kernels.h -- launch descriptors shared by the host API (fa_api.cpp) and
// the kernel translation units.  Plain structs of device pointers and sizes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Split-KV decode, stage 1 (and the single-split path that finishes in place).
struct DecodeArgs {
    const uint16_t* q;        // [B][Q_N][D] (q_seq == 1: both layouts coincide)
    const uint16_t* k;
    const uint16_t* v;
    const int64_t* lens;      // [B] or null
    float* o_part;            // [B][Q_N][splits][D]
    float* m_part;            // [B][Q_N][splits]
    float* l_part;
    void* out;                // single-split path: [B][Q_N][D]
    float* lse;               // single-split path: [B][Q_N] or null
    int64_t kv_seq;
    int64_t chunk;            // tokens per split (multiple of 64)
    int64_t kv_stride_s;      // elements between consecutive tokens of one head
    int64_t kv_stride_n;      // elements between KV heads
    int64_t kv_stride_b;      // elements between batches (contiguous cache)
    // Paged cache (block_table non-null): token j of batch b is row j % block_size
    // of physical block block_table[b * max_blocks + j / block_size]; kv_stride_s
    // and kv_stride_n then step inside a block, kv_stride_blk between blocks.
    const int32_t* block_table;
    int64_t kv_stride_blk;
    int32_t block_size;
    int32_t max_blocks;
    int32_t num_blocks;
    // Fused plan: [units] counters (units = B * KV_N * head_groups), zero on
    // entry and left zero; out / lse then receive the merged result.
    unsigned* counters;
    int32_t num_splits;
    int32_t num_heads;        // Q_N
    int32_t num_kv_heads;     // KV_N
    int32_t group;            // g = Q_N / KV_N
    int32_t head_groups;      // workgroups per KV head along g
    float scale_log2;         // scale * log2(e)
    // Matrix-core stage 1 only: a length-balanced schedule (bal_nwg > 0, see
    // bal_locate) instead of num_splits fixed chunks; num_splits is then the
    // slot count per row of the partials.
    int32_t bal_nwg;
    int32_t batch;            // B (read by the balanced schedule)
    // Query positions and masks (matrix-core stage 1 only; zero / null for
    // one query position without a mask).  Partial and output rows are
    // (b, n1, i) = (b * Q_N + n1) * q_seq + i; the g * q_seq rows of a KV head
    // (head-major: h * q_seq + i) fill row_groups tiles of 32 rows.
    int64_t q_seq;            // Q_S >= 1
    int64_t q_stride_s, q_stride_n, q_stride_b;  // elements, q and out
    int32_t row_groups;       // ceil(group * q_seq / 32), 1..16
    int32_t out_bsnd;         // out rows in BSND order (else BNSD)
    const int32_t* used_q;    // [B] query positions in use (seqused_q), or null
    int32_t mask_mode;        // 0 none, 1 causal, 2 boolean tensor, 3 window
    int32_t mask_dword;       // boolean mask read 4 keys per load (aligned, key stride 1)
    const uint8_t* mask;
    int64_t mask_stride[4];   // (b, n1, i, j) element strides, 0 broadcasts
    int32_t win_left, win_right;  // window bounds, 0x7fffffff = unbounded
    int32_t zero_q;           // scale underflows to 0 in fp32: every score is 0
};

struct CombineArgs {
    const float* o_part;
    const float* m_part;
    const float* l_part;
    void* out;                // shape of q: row (b, n1, i) at ((b*Q_N+n1)*Q_S+i)*D (BNSD) or ((b*Q_S+i)*Q_N+n1)*D (BSND)
    float* lse;               // [B][Q_N][Q_S] or null
    int64_t rows;             // B * Q_N * Q_S
    int64_t q_seq;            // Q_S
    int32_t out_bsnd;
    int32_t num_splits;       // slots per row
    // Length-balanced plan (bal_nwg > 0): row (b, n1) holds the pieces of
    // batch b only, their count computed as the stage-1 kernel did.
    int32_t bal_nwg;
    const int64_t* lens;
    int64_t kv_seq;
    int32_t batch, num_heads, num_kv_heads;
};

struct PrefillArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    void* out;
    float* lse;               // [B][Q_N][Q_S] or null
    const int64_t* lens;
    const uint8_t* mask;
    int64_t mask_stride[4];
    int64_t q_seq, kv_seq;
    int64_t q_stride_s, q_stride_n, q_stride_b;    // elements
    int64_t kv_stride_s, kv_stride_n, kv_stride_b;
    int32_t num_heads, num_kv_heads, group;
    int32_t q_tiles;
    int32_t negate_q;         // 1 when scale < 0: q's sign is flipped, scale_log2 = |scale|*log2(e)
    float scale_log2;
    int32_t win_left;         // window mask: keys qrow - win_left .. qrow + win_right kept;
    int32_t win_right;        // 0x7fffffff = unbounded on that side
    int32_t zero_q;           // scale underflows to 0 in fp32: q is read as zeros (every score 0)
    int32_t mask_dwords;      // boolean tensor in runs of 4-byte aligned keys (see prefill_rows_per_tile)
    // Packed layout (work != null): sequence b spans q rows [cu_q[b], cu_q[b+1])
    // and kv rows [cu_kv[b], cu_kv[b+1]) of the [T][N][D] tensors; q_seq and
    // kv_seq are the totals.  The work list holds (sequence, q tile) pairs,
    // tiles of the kernel's 128 or 256 rows, heaviest first; sequence index `batch` stands for the rows past
    // the last sequence.  Entries (-1, -1) pad the list.
    const int32_t* cu_q;
    const int32_t* cu_kv;
    const int32_t* used_q;    // [batch] or null
    const int32_t* work;      // [work_items][2]
    int32_t work_items;
    int32_t batch;
    // Boolean mask staged through LDS (instantiation 3): an optional summary
    // of the mask (MaskSummaryArgs), cls_words words per (slice, q tile).
    const uint32_t* mask_cls;
    int32_t cls_words;
    // CUs of the device (the persistent launch's grid; set by the caller) and
    // the units of work (query tile, head, batch) the launch covers (set by
    // the launcher).
    int32_t cus;
    int64_t units;
};

// Summary of a boolean mask over the prefill's tiles of 128 query rows x 64
// keys.  Slice (sb, sn) is the mask at b = sb, n = sn (a broadcast dimension,
// stride 0, has one slice).  Each (slice, q tile) owns a row of `words` 32-bit
// words, word w covering KV tiles 16*w .. 16*w+15 with two bits per tile:
// bit 0 set when some key of the tile is visible to some query row of the
// tile, bit 1 set when some key is masked for some row.  A tile holding no
// key (past kv_seq) reads 0.  Entry (slice, qt, w) is at
// out[((sb * slices_n + sn) * q_tiles + qt) * words + w].
constexpr int kMaskRowsPerTile = 128;
constexpr int kMaskKeysPerTile = 64;
constexpr int kMaskTilesPerWord = 16;
struct MaskSummaryArgs {
    const uint8_t* mask;
    int64_t mask_stride[4];
    int64_t q_seq, kv_seq;    // kv_seq a multiple of 16, rows 16-byte aligned
    int32_t q_tiles, words, slices_n;
    int64_t blocks;           // slices * q_tiles * words
    uint32_t* out;
};

// Geometry of one packed sequence, with every offset clamped into its tensor.
struct SeqGeom {
    int64_t q0, q_full, q_used;  // first q row, rows owned, rows computed
    int64_t k0, kv_len;          // first kv row, keys visible (after truncation)
};

__device__ __forceinline__ SeqGeom seq_geometry(const int32_t* cu_q, const int32_t* cu_kv, const int32_t* used_q,
                                                const int64_t* lens, int64_t b, int64_t batch, int64_t q_total,
                                                int64_t kv_total) {
    auto clampi = [](int64_t x, int64_t lo, int64_t hi) { return x < lo ? lo : (x > hi ? hi : x); };
    SeqGeom g;
    if (b >= batch) {  // rows past the last sequence: owned, never computed
        g.q0 = clampi(cu_q[batch], 0, q_total);
        g.q_full = q_total - g.q0;
        g.q_used = 0;
        g.k0 = 0;
        g.kv_len = 0;
        return g;
    }
    g.q0 = clampi(cu_q[b], 0, q_total);
    g.q_full = clampi(cu_q[b + 1], g.q0, q_total) - g.q0;
    g.q_used = used_q ? clampi(used_q[b], 0, g.q_full) : g.q_full;
    g.k0 = clampi(cu_kv[b], 0, kv_total);
    g.kv_len = clampi(cu_kv[b + 1], g.k0, kv_total) - g.k0;
    if (lens) g.kv_len = clampi(lens[b], 0, g.kv_len);
    return g;
}

// Cost-ordered work list of a packed batch (one workgroup of 1024 threads).
struct VarlenScheduleArgs {
    const int32_t* cu_q;
    const int32_t* cu_kv;
    const int32_t* used_q;
    const int64_t* lens;
    int32_t* work;            // [capacity][2]
    int64_t q_total, kv_total;
    int32_t batch;
    int32_t capacity;
    int32_t mask_mode;        // prefill mask instantiation (1 causal, 4 window: fewer tiles)
    int32_t win_left, win_right;
    int32_t rows;             // query rows per tile of the prefill kernel that runs (128 or 256)
};
constexpr int kVarlenMaxBatch = 16383;

// Block ids one paged stage-1 workgroup stages in LDS: a chunk may touch at most
// this many blocks.
constexpr int kPagedTableLds = 1024;
// Block ids a one-wave matrix-core decode workgroup keeps in a register (one
// per lane): its paged chunks may span at most this many blocks.
constexpr int kLaneBlocks = 64;

// Largest split count the fused stage-1 merge handles (its weights sit in LDS).
constexpr int kFusedMaxSplits = 256;

// Launchers: return hipSuccess or the launch error.  dtype: 0 = fp16, 1 = bf16.
hipError_t launch_decode_stage1(const DecodeArgs& a, int dtype, int head_dim, int heads_per_wg,
                                bool finish, int64_t batch, hipStream_t stream);
// Stage-1 workgroups one CU holds at once for this instantiation, from the
// runtime's occupancy calculator; 0 when no device answers.
int decode_stage1_residency(int dtype, int head_dim, int heads_per_wg, bool paged, bool masked = false);
hipError_t launch_combine(const CombineArgs& a, int dtype, int head_dim, hipStream_t stream);
// Length-balanced decode schedule (matrix-core stage 1 with per-batch
// lengths).  Batch b has T_b = ceil(L_b / 64) tiles per KV head; with
// W = KV_N * sum_b T_b and a target of nwg workgroups, a piece holds
// tstar = max(1, ceil(W / nwg)) tiles and batch b has n_b = ceil(T_b / tstar)
// pieces per KV head, so every piece is about the same work whatever the
// lengths.  Workgroups are numbered batch-major, then KV head, then piece; at
// most nwg + B * KV_N of them are needed.  All lanes of a wave call these
// (the results are wave-uniform).
__device__ __forceinline__ int64_t bal_len(const int64_t* lens, int64_t b, int64_t kv_seq) {
    int64_t L = lens[b];
    return L < 0 ? 0 : (L > kv_seq ? kv_seq : L);
}
__device__ __forceinline__ int64_t bal_tstar(const int64_t* lens, int64_t batch, int64_t kv_seq, int32_t kv_heads,
                                             int32_t nwg) {
    const int lane = threadIdx.x & 63;
    long long w = 0;
    for (int64_t b = lane; b < batch; b += 64) w += (bal_len(lens, b, kv_seq) + 63) / 64;
    for (int off = 32; off > 0; off >>= 1) w += __shfl_xor(w, off, 64);
    const int64_t W = (int64_t)w * kv_heads;
    const int64_t t = (W + nwg - 1) / nwg;
    return t < 1 ? 1 : t;
}
__device__ __forceinline__ int64_t bal_pieces(const int64_t* lens, int64_t b, int64_t kv_seq, int64_t tstar) {
    const int64_t T = (bal_len(lens, b, kv_seq) + 63) / 64;
    return (T + tstar - 1) / tstar;
}
// Workgroup w -> (batch, KV head, piece, pieces of the batch); false when w
// is past the last piece.
__device__ __forceinline__ bool bal_locate(const int64_t* lens, int64_t batch, int64_t kv_seq, int32_t kv_heads,
                                           int64_t tstar, int64_t w, int64_t* b_out, int* n2_out, int64_t* j_out,
                                           int64_t* nb_out) {
    const int lane = threadIdx.x & 63;
    long long acc = 0;  // workgroups of the batches before this block of 64
    for (int64_t base = 0; base < batch; base += 64) {
        const int64_t b = base + lane;
        const long long cnt = b < batch ? (long long)bal_pieces(lens, b, kv_seq, tstar) * kv_heads : 0;
        long long x = cnt;  // inclusive scan over the lanes
        for (int off = 1; off < 64; off <<= 1) {
            const long long y = __shfl_up(x, off, 64);
            if (lane >= off) x += y;
        }
        const bool hit = cnt > 0 && w >= acc + (x - cnt) && w < acc + x;
        const unsigned long long m = __ballot(hit);
        if (m) {
            const int src = __builtin_ctzll(m);
            const long long start = acc + __shfl(x - cnt, src, 64);
            const long long nb = __shfl(cnt, src, 64) / kv_heads;
            const long long rem = (long long)w - start;
            *b_out = base + src;
            *n2_out = (int)(rem / nb);
            *j_out = rem % nb;
            *nb_out = nb;
            return true;
        }
        acc += __shfl(x, 63, 64);
    }
    return false;
}

// The same lookup from one load of the lengths when the batch fits a wave
// (lane b holds batch b's length; the tile total, the scan and the batch's
// length are then shuffles of it), so a workgroup starts with one memory round
// trip instead of one per helper above, and in 32-bit arithmetic with the
// uniform divisions done once on the scalar unit (a 64-bit division per lane
// is a long instruction sequence).  Also returns tstar and the batch's length
// L.  Falls back to the helpers above past 64 batches or 2^30 tiles of work.
struct BalWave {
    int32_t L;      // this lane's batch length (clamped), 0 past the batch
    int32_t T;      // its 64-key tiles
    int32_t tstar;  // tiles per piece (uniform)
    bool ok;        // the 32-bit form applies
};
__device__ __forceinline__ BalWave bal_wave(const int64_t* lens, int64_t batch, int64_t kv_seq, int32_t kv_heads,
                                            int32_t nwg) {
    BalWave r;
    r.ok = batch <= 64 && kv_seq < (int64_t(1) << 31);
    if (!r.ok) return r;
    const int lane = threadIdx.x & 63;
    r.L = lane < batch ? (int32_t)bal_len(lens, lane, kv_seq) : 0;
    r.T = (r.L + 63) >> 6;
    int tot = r.T;
    for (int off = 32; off > 0; off >>= 1) tot += __shfl_xor(tot, off, 64);
    const int64_t W = (int64_t)__builtin_amdgcn_readfirstlane(tot) * kv_heads;
    if (W >= (int64_t(1) << 30) || nwg <= 0) {
        r.ok = false;
        return r;
    }
    const uint32_t w32 = (uint32_t)W, n32 = (uint32_t)nwg;
    uint32_t t = (w32 + n32 - 1) / n32;
    r.tstar = (int32_t)(t < 1 ? 1 : t);
    return r;
}
__device__ __forceinline__ bool bal_find(const int64_t* lens, int64_t batch, int64_t kv_seq, int32_t kv_heads,
                                         int32_t nwg, int64_t w, int64_t* tstar_out, int64_t* b_out, int* n2_out,
                                         int64_t* j_out, int64_t* L_out) {
    const BalWave bw = bal_wave(lens, batch, kv_seq, kv_heads, nwg);
    if (!bw.ok) {
        const int64_t tstar = bal_tstar(lens, batch, kv_seq, kv_heads, nwg);
        int64_t nb;
        if (!bal_locate(lens, batch, kv_seq, kv_heads, tstar, w, b_out, n2_out, j_out, &nb)) return false;
        *tstar_out = tstar;
        *L_out = bal_len(lens, *b_out, kv_seq);
        return true;
    }
    const int lane = threadIdx.x & 63;
    const uint32_t ts = (uint32_t)bw.tstar;
    const int cnt = (int)(((uint32_t)bw.T + ts - 1) / ts) * kv_heads;  // this batch's workgroups
    int x = cnt;  // inclusive scan over the lanes
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    const bool hit = cnt > 0 && w >= x - cnt && w < x;
    const unsigned long long m = __ballot(hit);
    if (!m) return false;
    const int src = __builtin_ctzll(m);
    const uint32_t start = (uint32_t)__builtin_amdgcn_readfirstlane(__shfl(x - cnt, src, 64));
    const uint32_t nb = (uint32_t)__builtin_amdgcn_readfirstlane(__shfl(cnt, src, 64)) / (uint32_t)kv_heads;
    const uint32_t rem = (uint32_t)w - start;
    *tstar_out = bw.tstar;
    *b_out = src;
    *n2_out = (int)(rem / nb);
    *j_out = rem % nb;
    *L_out = __builtin_amdgcn_readfirstlane(__shfl(bw.L, src, 64));
    return true;
}
// Pieces of batch b under the plan, from one load of the lengths as above.
__device__ __forceinline__ int64_t bal_row_pieces(const int64_t* lens, int64_t batch, int64_t kv_seq,
                                                  int32_t kv_heads, int32_t nwg, int64_t b) {
    const BalWave bw = bal_wave(lens, batch, kv_seq, kv_heads, nwg);
    if (!bw.ok) return bal_pieces(lens, b, kv_seq, bal_tstar(lens, batch, kv_seq, kv_heads, nwg));
    const uint32_t Tb = (uint32_t)__builtin_amdgcn_readfirstlane(__shfl(bw.T, (int)b, 64));
    return (Tb + (uint32_t)bw.tstar - 1) / (uint32_t)bw.tstar;
}

// Matrix-core stage 1 for grouped heads (1 <= group <= 32, contiguous or
// paged cache with block sizes a multiple of 16, head_dim 64 or 128): one
// workgroup per (batch, KV head, split), the same partial layout as
// launch_decode_stage1 (finish = one-split plan writing out and lse).  waves
// = 2: two waves share 64-key tiles and merge at the end; waves = 1: one wave
// per workgroup on 32-key tiles, a quarter of the LDS, so more workgroups
// (and more tile loads) per CU for short pieces.
int decode_mfma_residency(int dtype, int head_dim, bool paged, int waves);
hipError_t launch_decode_mfma(const DecodeArgs& a, int dtype, int head_dim, bool finish, int waves, int64_t batch,
                              hipStream_t stream);
// Query rows per prefill workgroup: 256 on the interleaved kernel (D = 128;
// a boolean tensor not staged in 16-byte runs needs runs of 4-byte aligned
// keys, mask_dwords), else 128.
int prefill_rows_per_tile(int head_dim, int mask_mode, bool mask_dwords);
bool prefill_interleaved(int head_dim, int mask_mode, bool mask_dwords);
// Workgroups of a persistent interleaved launch (one per CU, a multiple of 8,
// each taking units in turn), or 0 when the launch is one workgroup per unit:
// head dim 128 without a mask, with a window or causal, more units than CUs
// (on the packed layout, entries x heads).
int64_t prefill_persistent_grid(int head_dim, int mask_mode, int64_t units, int cus);
hipError_t launch_prefill(const PrefillArgs& a, int dtype, int head_dim, int mask_mode,
                          int64_t batch, hipStream_t stream);
hipError_t launch_varlen_schedule(const VarlenScheduleArgs& a, hipStream_t stream);
hipError_t launch_mask_summary(const MaskSummaryArgs& a, hipStream_t stream);

}  // namespace fa
