// fa_decode.hip -- split-KV decode for gfx950: stage 1 (per-chunk partial
// softmax statistics and unnormalised output) and stage 2 (the LSE combine).
//
// Stage 1 follows the FlashDecoding tutorial (section 3.2): each workgroup owns
// one KV chunk of one KV head, keeps the query resident, streams the chunk's K
// and V rows once, and writes O_c = sum_j exp(s_j - m_c) v_j (not divided by
// l_c) together with m_c and l_c.  Stage 2 merges the chunks with the FD
// reduction of the FlashAttn developer guide (section 10).
//
// Decode reads every cached K/V byte once and does ~2 FMAs per byte, so it is
// bound by HBM bandwidth.  The kernel is laid out for that: D/8 lanes cover one
// 16-byte-per-lane KV row, so one wave load instruction reads 2 (D=256), 4
// (D=128) or 8 (D=64) whole rows = 1 KiB contiguous in the BNSD layout; the K and V of
// the next two iterations are in flight while the current rows are consumed; the
// dot product is reduced across the row's lanes with DPP moves.  Each lane
// group (the lanes of one row slot) keeps its own running max / sum / output,
// so the streaming loop has no cross-group traffic; groups and waves are
// merged once at the end.  The g query heads that share a KV head (GQA) are
// processed by the same workgroup so their K/V rows are read once.
//
// Fused split-KV (one launch): after writing its chunk's partials with
// device-coherent stores a workgroup counts itself done on a per-unit counter
// (a vector atomic on global memory), and the workgroup that completes the
// count merges that unit's rows with the FD reduction right away and resets
// the counter, so no second kernel waits for the whole grid.  This takes the
// place of the pages' SyncAll between the split and the reduction (FlashAttn
// developer guide, FA/FD overlap): rows are merged as soon as their own
// chunks finish.
//
// With a paged cache (FlashAttn developer guide 1.2, PagedAttention) the
// workgroup first stages the physical block ids of its chunk in LDS; every lane
// then follows its row slots block by block with an incrementally advanced
// (block, row) cursor, so the streaming loop adds one LDS read and one address
// multiply per row and no division.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

// Stage-1 output modes: partials only, the final output of a one-split plan,
// or partials plus the in-kernel merge of the fused plan.
constexpr int kPartial = 0, kFinish = 1, kFused = 2;

// MASKED: a boolean mask tensor (one query position; contiguous cache): the
// mask byte of each key and query head is loaded with the key's K/V row, and
// a masked key's score is -inf.
template <typename ST, int D, int GH, int MODE, bool PAGED, bool MASKED = false>
__global__ __launch_bounds__(256) void decode_stage1_kernel(DecodeArgs a) {
    static_assert(!(MASKED && (PAGED || MODE == 2)), "masked: contiguous cache, partial or finish");
    constexpr int LPR = D / 8;     // lanes per KV row
    constexpr int RPL = 64 / LPR;  // rows per wave load
    constexpr int U = 2;                   // row slots per lane per iteration
    constexpr int DEPTH = (GH >= 4) ? 1 : 2;  // iterations of K/V loads in flight ahead
    // (both chosen so the common instantiations stay within 128 VGPRs: four
    // workgroups per CU, the residency the split plan assumes)
    constexpr int TW = RPL * U;    // tokens per wave iteration
    constexpr int NW = 4;          // waves per workgroup

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int sub = lane % LPR;
    const int grp = lane / LPR;

    const int64_t blk = blockIdx.x;
    const int split = (int)(blk % a.num_splits);
    const int64_t unit = blk / a.num_splits;
    const int hg = (int)(unit % a.head_groups);
    const int64_t bn2 = unit / a.head_groups;
    const int n2 = (int)(bn2 % a.num_kv_heads);
    const int64_t b = bn2 / a.num_kv_heads;

    int64_t L = a.kv_seq;
    if (a.lens) {
        L = a.lens[b];
        L = L < 0 ? 0 : (L > a.kv_seq ? a.kv_seq : L);
    }
    const int64_t c0 = (int64_t)split * a.chunk;
    int64_t c1 = c0 + a.chunk;
    if (c1 > L) c1 = L;

    if (c1 > c0) {
        // Resident query slice, kept in its 16-bit storage form: q.k is taken with
        // packed two-element dot products (fp32 accumulation) straight on the
        // loaded K words, and the score is scaled by scale*log2(e) afterwards.
        u32x4 qp[GH];
#pragma unroll
        for (int h = 0; h < GH; ++h) {
            const int gi = hg * GH + h;
            qp[h] = u32x4{0u, 0u, 0u, 0u};
            if (gi < a.group && !a.zero_q) {  // zero_q: scale 0, every score 0
                const int64_t n1 = (int64_t)n2 * a.group + gi;
                qp[h] = ld128(a.q + (b * a.num_heads + n1) * D + sub * 8);
            }
        }
        const float c = a.scale_log2;

        // Per lane group and query head: a reference max m (scores are
        // exponentiated against it and it moves only when a score exceeds it by
        // more than 2^kTau), the true running max tm, the sum l and the output.
        constexpr float kTau = 8.f;
        float m[GH], tm[GH], l[GH], acc[GH][8];
#pragma unroll
        for (int h = 0; h < GH; ++h) {
            m[h] = kNegInf;
            tm[h] = kNegInf;
            l[h] = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
        }

        const int64_t head_off = (PAGED ? 0 : b * a.kv_stride_b) + (int64_t)n2 * a.kv_stride_n + sub * 8;
        const uint16_t* kb = a.k + head_off;
        const uint16_t* vb = a.v + head_off;
        const int64_t ss = a.kv_stride_s;

        // Contiguous cache: one buffer resource per tensor, based at this head's
        // first row of the chunk and ending after its last valid row, so rows at
        // or past the length load as zeros without a branch and each load takes
        // a 32-bit offset (the host keeps (chunk + 256) rows below 2^31 bytes).
        const int row_bytes = (int)(ss * 2);
        const int64_t rbase = PAGED ? 0 : b * a.kv_stride_b + (int64_t)n2 * a.kv_stride_n + c0 * ss;
        const int nrec = (!PAGED && c1 > c0) ? (int)((c1 - c0) * ss * 2) : 0;
        const buf_rsrc rk = make_rsrc(a.k + rbase, nrec);  // unused by the paged instantiation
        const buf_rsrc rv = make_rsrc(a.v + rbase, nrec);

        // Paged cache: block ids of the chunk's logical blocks [cb, cb + nblk),
        // clamped into the physical range, and per-slot (block, row) cursors that
        // follow the positions load() is called with (t0 + k*NW*TW, k = 0, 1, ...).
        __shared__ int32_t s_blk[PAGED ? kPagedTableLds : 1];
        int pb[U], pr[U];
        int step_q = 0, step_r = 0;
        if constexpr (PAGED) {
            const int bs = a.block_size;
            const int64_t cb = c0 / bs;
            const int64_t nblk = (c1 > c0) ? (c1 - 1) / bs - cb + 1 : 0;
            const int32_t* tb = a.block_table + b * a.max_blocks + cb;
            for (int i = threadIdx.x; i < nblk; i += 256) {
                int32_t id = tb[i];
                id = id < 0 ? 0 : (id >= a.num_blocks ? a.num_blocks - 1 : id);
                s_blk[i] = id;
            }
            __syncthreads();
            const int rel0 = (int)(c0 - cb * bs) + wave * TW + grp;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                pb[u] = (rel0 + u * RPL) / bs;
                pr[u] = (rel0 + u * RPL) % bs;
            }
            step_q = (NW * TW) / bs;
            step_r = (NW * TW) % bs;
        }

        // Mask rows (query position 0, unit key stride) of the workgroup's
        // query heads from the chunk's first key; a lane's U bytes per head
        // are packed into one word, byte u for row slot u.
        const uint8_t* mrow[GH];
#pragma unroll
        for (int h = 0; h < GH; ++h) {
            const int64_t n1 = (int64_t)n2 * a.group + hg * GH + h;
            mrow[h] = MASKED ? a.mask + b * a.mask_stride[0] + n1 * a.mask_stride[1] + c0 : nullptr;
        }
        auto load = [&](int64_t t0, u32x4* kw, u32x4* vw, uint32_t* mw) __attribute__((always_inline)) {
            if constexpr (MASKED) {
#pragma unroll
                for (int h = 0; h < GH; ++h) mw[h] = 0u;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t t = t0 + u * RPL + grp;
                if constexpr (MASKED) {
                    const int rel = (int)(t - c0);
#pragma unroll
                    for (int h = 0; h < GH; ++h)
                        mw[h] |= ((t < c1) ? (uint32_t)(mrow[h][rel] != 0) : 1u) << (8 * u);
                }
                if constexpr (!PAGED) {
                    const int voff = (int)(t - c0) * row_bytes + sub * 16;
                    kw[u] = buf_ld128(rk, voff);
                    vw[u] = buf_ld128(rv, voff);
                } else if (t < c1) {
                    const int64_t off = (int64_t)s_blk[pb[u]] * a.kv_stride_blk + (int64_t)pr[u] * ss;
                    kw[u] = ld128_stream(kb + off);
                    vw[u] = ld128_stream(vb + off);
                } else {
                    kw[u] = u32x4{0u, 0u, 0u, 0u};
                    vw[u] = u32x4{0u, 0u, 0u, 0u};
                }
                if constexpr (PAGED) {
                    pb[u] += step_q;
                    pr[u] += step_r;
                    if (pr[u] >= a.block_size) {
                        pr[u] -= a.block_size;
                        pb[u] += 1;
                    }
                }
            }
        };

        // One iteration: the rows at t0 (+ slot and group offsets) are in (kw, vw).
        auto consume = [&](int64_t t0, const u32x4* kw, const u32x4* vw, const uint32_t* mw)
                           __attribute__((always_inline)) {
            float vf[U][8];
#pragma unroll
            for (int u = 0; u < U; ++u) unpack8<ST>(vw[u], vf[u]);
#pragma unroll
            for (int h = 0; h < GH; ++h) {
                float s[U];
                float mx = kNegInf;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    float part = dot8<ST>(qp[h], kw[u]);
                    part = group_sum<LPR>(part) * c;
                    bool keep = t0 + u * RPL + grp < c1;
                    if constexpr (MASKED) keep = keep && ((mw[h] >> (8 * u)) & 0xffu) == 0u;
                    s[u] = keep ? part : kNegInf;
                    mx = fmaxf(mx, s[u]);
                }
                tm[h] = fmaxf(tm[h], mx);
                if (mx > m[h] + kTau) {  // rare after the first rows: rescale to the new reference
                    const float alpha = fast_exp2(m[h] - mx);
                    l[h] *= alpha;
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
                    m[h] = mx;
                }
                const float ms = (m[h] == kNegInf) ? 0.f : m[h];
                float psum = 0.f;
                float p[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    p[u] = fast_exp2(s[u] - ms);
                    psum += p[u];
                }
                l[h] += psum;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float x = acc[h][e];
#pragma unroll
                    for (int u = 0; u < U; ++u) x = __builtin_fmaf(p[u], vf[u][e], x);
                    acc[h][e] = x;
                }
            }
        };

        // Ring of DEPTH + 1 load buffers: the loop is unrolled over the ring so
        // every buffer keeps a fixed role (no register rotation), and the rows
        // DEPTH iterations ahead are in flight while one is consumed.
        constexpr int64_t STEP = NW * TW;
        int64_t t0 = c0 + (int64_t)wave * TW;
        u32x4 kA[U], vA[U], kB[U], vB[U];
        constexpr int MW = MASKED ? GH : 1;
        uint32_t mA[MW], mB[MW], mC[MW];
        load(t0, kA, vA, mA);
        if constexpr (DEPTH == 1) {
            while (true) {
                if (t0 >= c1) break;
                load(t0 + STEP, kB, vB, mB);
                consume(t0, kA, vA, mA);
                t0 += STEP;
                if (t0 >= c1) break;
                load(t0 + STEP, kA, vA, mA);
                consume(t0, kB, vB, mB);
                t0 += STEP;
            }
        } else {
            u32x4 kC[U], vC[U];
            load(t0 + STEP, kB, vB, mB);
            while (true) {
                if (t0 >= c1) break;
                load(t0 + 2 * STEP, kC, vC, mC);
                consume(t0, kA, vA, mA);
                t0 += STEP;
                if (t0 >= c1) break;
                load(t0 + 2 * STEP, kA, vA, mA);
                consume(t0, kB, vB, mB);
                t0 += STEP;
                if (t0 >= c1) break;
                load(t0 + 2 * STEP, kB, vB, mB);
                consume(t0, kC, vC, mC);
                t0 += STEP;
            }
        }

        // Move each lane group from its reference max to the true max, then merge
        // the row-slot groups of this wave (lanes that share `sub`).
#pragma unroll
        for (int h = 0; h < GH; ++h) {
            if (tm[h] != kNegInf && tm[h] != m[h]) {
                const float f = fast_exp2(m[h] - tm[h]);
                l[h] *= f;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] *= f;
            }
            m[h] = tm[h];
            float M = m[h];
#pragma unroll
            for (int off = LPR; off < 64; off <<= 1) M = fmaxf(M, shfl_xor(M, off));
            const float ms = (M == kNegInf) ? 0.f : M;
            const float f = fast_exp2(m[h] - ms);
            float lw = l[h] * f;
#pragma unroll
            for (int off = LPR; off < 64; off <<= 1) lw += shfl_xor(lw, off);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float x = acc[h][e] * f;
#pragma unroll
                for (int off = LPR; off < 64; off <<= 1) x += shfl_xor(x, off);
                acc[h][e] = x;
            }
            m[h] = M;
            l[h] = lw;
        }

        // Merge the waves through LDS and write the chunk's result.
        __shared__ float s_m[NW][GH];
        __shared__ float s_l[NW][GH];
        __shared__ float s_acc[NW][GH][D];
        if (grp == 0) {
#pragma unroll
            for (int h = 0; h < GH; ++h)
#pragma unroll
                for (int e = 0; e < 8; ++e) s_acc[wave][h][sub * 8 + e] = acc[h][e];
        }
        if (lane == 0) {
#pragma unroll
            for (int h = 0; h < GH; ++h) {
                s_m[wave][h] = m[h];
                s_l[wave][h] = l[h];
            }
        }
        __syncthreads();

        for (int idx = threadIdx.x; idx < GH * D; idx += 256) {
            const int h = idx / D;
            const int d = idx % D;
            const int gi = hg * GH + h;
            if (gi >= a.group) continue;
            float M = kNegInf;
#pragma unroll
            for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w][h]);
            const float ms = (M == kNegInf) ? 0.f : M;
            float Lt = 0.f, A = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const float f = fast_exp2(s_m[w][h] - ms);
                Lt = __builtin_fmaf(s_l[w][h], f, Lt);
                A = __builtin_fmaf(s_acc[w][h][d], f, A);
            }
            const int64_t row = b * a.num_heads + (int64_t)n2 * a.group + gi;
            if constexpr (MODE == kFinish) {
                const bool empty = (M == kNegInf);
                uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
                out[row * D + d] = to_bits<ST>(empty ? 0.f : A / Lt);
                if (d == 0 && a.lse) a.lse[row] = empty ? kPosInf : (M + log2f(Lt)) * kLn2;
            } else {
                const int64_t slot = row * a.num_splits + split;
                const float mo = (M == kNegInf) ? kNegInf : M * kLn2;
                if constexpr (MODE == kFused) {  // device-coherent stores: another CU's L2 may merge them
                    __hip_atomic_store(a.o_part + slot * D + d, A, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    if (d == 0) {
                        __hip_atomic_store(a.m_part + slot, mo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        __hip_atomic_store(a.l_part + slot, Lt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                } else {
                    a.o_part[slot * D + d] = A;
                    if (d == 0) {
                        a.m_part[slot] = mo;
                        a.l_part[slot] = Lt;
                    }
                }
            }
        }
    } else {
        // A chunk at or past the length: its empty partial (or the row
        // defaults of a one-split plan) without touching K or V.
        for (int idx = threadIdx.x; idx < GH * D; idx += 256) {
            const int h = idx / D;
            const int d = idx % D;
            const int gi = hg * GH + h;
            if (gi >= a.group) continue;
            const int64_t row = b * a.num_heads + (int64_t)n2 * a.group + gi;
            if constexpr (MODE == kFinish) {
                reinterpret_cast<uint16_t*>(a.out)[row * D + d] = 0;
                if (d == 0 && a.lse) a.lse[row] = kPosInf;
            } else {
                const int64_t slot = row * a.num_splits + split;
                if constexpr (MODE == kFused) {
                    __hip_atomic_store(a.o_part + slot * D + d, 0.f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    if (d == 0) {
                        __hip_atomic_store(a.m_part + slot, kNegInf, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        __hip_atomic_store(a.l_part + slot, 0.f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                } else {
                    a.o_part[slot * D + d] = 0.f;
                    if (d == 0) {
                        a.m_part[slot] = kNegInf;
                        a.l_part[slot] = 0.f;
                    }
                }
            }
        }
    }

    if constexpr (MODE == kFused) {
        // Count this chunk and let the workgroup that completes the unit's
        // count merge its rows.  Every wave's partial stores complete before
        // the barrier; thread 0 then counts with a release at device (agent)
        // scope, which writes this XCD's L2 back to the point where the other
        // XCDs read, so the partials are visible device-wide before the count
        // moves.  Only the workgroup that completes the count acquires (drops
        // lines its caches may hold stale) before reading the other
        // workgroups' partials: a full fence in every workgroup, which also
        // invalidates each XCD's L2 each time, measured several times slower.
        __shared__ int s_last;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (threadIdx.x == 0) {
            const bool last = __hip_atomic_fetch_add(a.counters + unit, 1u, __ATOMIC_RELEASE,
                                                     __HIP_MEMORY_SCOPE_AGENT) == (unsigned)(a.num_splits - 1);
            if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            s_last = last;
        }
        __syncthreads();
        if (!s_last) return;
        // Every chunk of the unit has counted: leave the counter at zero for
        // the next call on this workspace.
        if (threadIdx.x == 0) __hip_atomic_store(a.counters + unit, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        auto ld = [](const float* p) __attribute__((always_inline)) {
            return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        };

        const int S = a.num_splits;
        __shared__ float s_w[GH][kFusedMaxSplits];
        __shared__ float s_inv[GH], s_lse[GH];
        // Weights: one wave per query head, each lane's m and l loads issued
        // together (S <= 256: up to four per lane).
        for (int h = wave; h < GH; h += NW) {
            const int gi = hg * GH + h;
            if (gi >= a.group) continue;
            const int64_t row = b * a.num_heads + (int64_t)n2 * a.group + gi;
            const float* mp = a.m_part + row * S;
            const float* lp = a.l_part + row * S;
            float mv[kFusedMaxSplits / 64], lv[kFusedMaxSplits / 64];
#pragma unroll
            for (int j = 0; j < kFusedMaxSplits / 64; ++j) {
                const int i = lane + 64 * j;
                mv[j] = (i < S) ? ld(mp + i) : kNegInf;
                lv[j] = (i < S) ? ld(lp + i) : 0.f;
            }
            float mx = kNegInf;
#pragma unroll
            for (int j = 0; j < kFusedMaxSplits / 64; ++j) mx = fmaxf(mx, mv[j]);
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, shfl_xor(mx, off));
            const float mx2 = mx * kLog2e;
            float ls = 0.f;
#pragma unroll
            for (int j = 0; j < kFusedMaxSplits / 64; ++j) {
                const int i = lane + 64 * j;
                const float w = (mv[j] == kNegInf) ? 0.f : fast_exp2(__builtin_fmaf(mv[j], kLog2e, -mx2));
                if (i < S) s_w[h][i] = w;
                ls = __builtin_fmaf(w, lv[j], ls);
            }
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) ls += shfl_xor(ls, off);
            if (lane == 0) {
                s_inv[h] = (mx == kNegInf) ? 0.f : 1.f / ls;
                s_lse[h] = (mx == kNegInf) ? kPosInf : mx + logf(ls);
            }
        }
        __syncthreads();
        // Outputs: TPO threads per (head, column), each summing a share of the
        // splits with 16 loads in flight at a time; shares meet in LDS.
        constexpr int OUTS = GH * D;
        constexpr int TPO = (OUTS >= 256) ? 1 : 256 / OUTS;
        __shared__ float s_part[(TPO > 1) ? 256 : 1];
        uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
        for (int idx = threadIdx.x; idx < OUTS * TPO; idx += 256) {
            const int o = idx % OUTS;
            const int share = idx / OUTS;
            const int h = o / D;
            const int d = o % D;
            const int gi = hg * GH + h;
            float A = 0.f;
            if (gi < a.group) {
                const int64_t row = b * a.num_heads + (int64_t)n2 * a.group + gi;
                const float* op = a.o_part + row * (int64_t)S * D + d;
                for (int i0 = share * 16; i0 < S; i0 += 16 * TPO) {
                    float ov[16];
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const int i = i0 + j;
                        ov[j] = (i < S && s_w[h][i] != 0.f) ? ld(op + (int64_t)i * D) : 0.f;  // empty chunks skipped
                    }
#pragma unroll
                    for (int j = 0; j < 16; ++j)
                        if (i0 + j < S) A = __builtin_fmaf(s_w[h][i0 + j], ov[j], A);
                }
            }
            if constexpr (TPO > 1) {
                s_part[idx] = A;
            } else if (gi < a.group) {
                const int64_t row = b * a.num_heads + (int64_t)n2 * a.group + gi;
                out[row * D + d] = to_bits<ST>(A * s_inv[h]);
                if (d == 0 && a.lse) a.lse[row] = s_lse[h];
            }
        }
        if constexpr (TPO > 1) {
            __syncthreads();
            if (threadIdx.x < OUTS) {
                const int o = threadIdx.x;
                const int h = o / D;
                const int d = o % D;
                const int gi = hg * GH + h;
                if (gi < a.group) {
                    float A = 0.f;
#pragma unroll
                    for (int t = 0; t < TPO; ++t) A += s_part[t * OUTS + o];
                    const int64_t row = b * a.num_heads + (int64_t)n2 * a.group + gi;
                    out[row * D + d] = to_bits<ST>(A * s_inv[h]);
                    if (d == 0 && a.lse) a.lse[row] = s_lse[h];
                }
            }
        }
    }
}



// Stage 2: one workgroup of 256 threads per (b, n1) row merges num_splits
// partials.  Thread t owns four head-dim columns (t % (D/4)) of one split group
// (t / (D/4)).  Its first partial-output loads, the row's m and l, and (for a
// length-balanced plan) the batch lengths are all issued before anything is
// reduced, so the common case -- a few dozen splits -- costs one memory
// latency plus the block reductions; slots past the row's piece count (stale
// in a balanced plan) are loaded but never weighted.
constexpr int kCombineWeightsLds = 2048;
constexpr int kCombinePreload = 4;  // partial-output loads per thread issued up front

__device__ __forceinline__ float block_max256(float x, float* red) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, shfl_xor(x, off));
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = x;
    __syncthreads();
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__device__ __forceinline__ float block_sum256(float x, float* red) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += shfl_xor(x, off);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = x;
    __syncthreads();
    return (red[0] + red[1]) + (red[2] + red[3]);
}

template <typename ST, int D>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
    constexpr int NQ = D / 4;      // float4 columns per row
    constexpr int NG = 256 / NQ;   // split groups
    __shared__ float red[4];
    __shared__ float s_w[kCombineWeightsLds];
    __shared__ f32x4 s_acc[NG][NQ];

    const int64_t row = blockIdx.x;
    const int t = threadIdx.x;
    const int dq = t % NQ;
    const int sg = t / NQ;
    const int SS = a.num_splits;  // slots per row
    const float* mp = a.m_part + row * SS;
    const float* lp = a.l_part + row * SS;
    const float* op = a.o_part + row * (int64_t)SS * D;
    // Row (b, n1, i) = (b * Q_N + n1) * Q_S + i; in BSND its output is at
    // ((b * Q_S + i) * Q_N + n1) * D (the same place when Q_S == 1).
    int64_t orow = row;
    if (a.out_bsnd && a.q_seq > 1) {
        const int64_t i = row % a.q_seq, bn = row / a.q_seq;
        orow = ((bn / a.num_heads) * a.q_seq + i) * a.num_heads + bn % a.num_heads;
    }
    uint16_t* out = reinterpret_cast<uint16_t*>(a.out) + orow * D;

    // Loads that need nothing else first: slot t's m and l, and this thread's
    // first kCombinePreload partial outputs.  Indexes past the row's slots
    // re-read its last slot (unbranched loads stay in flight together); those
    // values are never used.
    const int tc = t < SS ? t : SS - 1;
    const float m_t = mp[tc];
    const float l_t = lp[tc];
    f32x4 o_pre[kCombinePreload];
#pragma unroll
    for (int u = 0; u < kCombinePreload; ++u) {
        int i = sg + u * NG;
        i = i < SS ? i : SS - 1;
        o_pre[u] = *reinterpret_cast<const f32x4*>(op + (int64_t)i * D + 4 * dq);
    }
    int S = SS;                   // slots this row uses
    if (a.bal_nwg > 0) {          // length-balanced plan: the pieces of this row's batch
        const int64_t nb = bal_row_pieces(a.lens, a.batch, a.kv_seq, a.num_kv_heads, a.bal_nwg, row / a.num_heads);
        S = (int)(nb < SS ? nb : SS);
    }

    float mx = t < S ? m_t : kNegInf;
    for (int i = t + 256; i < S; i += 256) mx = fmaxf(mx, mp[i]);
    mx = block_max256(mx, red);
    if (mx == kNegInf) {  // every split empty: RowInvalid defaults
        if (t < NQ) {
            u32x2 z;
            z[0] = 0u;
            z[1] = 0u;
            *reinterpret_cast<u32x2*>(out + 4 * t) = z;
        }
        if (t == 0 && a.lse) a.lse[row] = kPosInf;
        return;
    }
    const float mx2 = mx * kLog2e;
    auto weight = [&](float mi) __attribute__((always_inline)) {
        return (mi == kNegInf) ? 0.f : fast_exp2(__builtin_fmaf(mi, kLog2e, -mx2));
    };
    float ls = 0.f;
    if (t < S) {
        const float w = weight(m_t);
        if (t < kCombineWeightsLds) s_w[t] = w;
        ls = w * l_t;
    }
    for (int i = t + 256; i < S; i += 256) {
        const float w = weight(mp[i]);
        if (i < kCombineWeightsLds) s_w[i] = w;
        ls = __builtin_fmaf(w, lp[i], ls);
    }
    ls = block_sum256(ls, red);  // its barriers also publish s_w

    auto w_of = [&](int i) __attribute__((always_inline)) {
        return i < kCombineWeightsLds ? s_w[i] : weight(mp[i]);
    };
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < kCombinePreload; ++u) {
        const int i = sg + u * NG;
        if (i < S) {
            const float w = w_of(i);
            if (w != 0.f) acc += w * o_pre[u];  // empty splits are skipped whatever their O holds
        }
    }
#pragma unroll 4
    for (int i = sg + kCombinePreload * NG; i < S; i += NG) {
        const f32x4 o = *reinterpret_cast<const f32x4*>(op + (int64_t)i * D + 4 * dq);
        const float w = w_of(i);
        if (w != 0.f) acc += w * o;
    }
    s_acc[sg][dq] = acc;
    __syncthreads();
    if (t < NQ) {
        f32x4 sum = s_acc[0][t];
#pragma unroll
        for (int g = 1; g < NG; ++g) sum += s_acc[g][t];
        const float inv = 1.f / ls;
        u32x2 w;
        w[0] = pack2<ST>(sum[0] * inv, sum[1] * inv);
        w[1] = pack2<ST>(sum[2] * inv, sum[3] * inv);
        *reinterpret_cast<u32x2*>(out + 4 * t) = w;
        if (t == 0 && a.lse) a.lse[row] = mx + logf(ls);
    }
}

template <typename ST, int D, int GH, bool PAGED>
static hipError_t dispatch_stage1_fin(const DecodeArgs& a, bool finish, int64_t blocks, hipStream_t s) {
    const dim3 grid((unsigned)blocks);
    if (finish) {
        hipLaunchKernelGGL((decode_stage1_kernel<ST, D, GH, kFinish, PAGED>), grid, dim3(256), 0, s, a);
    } else if (a.counters) {
        hipLaunchKernelGGL((decode_stage1_kernel<ST, D, GH, kFused, PAGED>), grid, dim3(256), 0, s, a);
    } else {
        hipLaunchKernelGGL((decode_stage1_kernel<ST, D, GH, kPartial, PAGED>), grid, dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

template <typename ST, int D, int GH>
static hipError_t dispatch_stage1(const DecodeArgs& a, bool finish, int64_t blocks, hipStream_t s) {
    if (a.mask) {  // boolean mask: contiguous cache, partials or the finished output
        if (a.block_table || a.counters) return hipErrorInvalidValue;
        const dim3 grid((unsigned)blocks);
        if (finish)
            hipLaunchKernelGGL((decode_stage1_kernel<ST, D, GH, kFinish, false, true>), grid, dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((decode_stage1_kernel<ST, D, GH, kPartial, false, true>), grid, dim3(256), 0, s, a);
        return hipGetLastError();
    }
    if (a.block_table) return dispatch_stage1_fin<ST, D, GH, true>(a, finish, blocks, s);
    return dispatch_stage1_fin<ST, D, GH, false>(a, finish, blocks, s);
}

template <typename ST, int D>
static hipError_t dispatch_stage1_gh(const DecodeArgs& a, int gh, bool finish, int64_t blocks, hipStream_t s) {
    switch (gh) {
        case 1: return dispatch_stage1<ST, D, 1>(a, finish, blocks, s);
        case 2: return dispatch_stage1<ST, D, 2>(a, finish, blocks, s);
        case 4: return dispatch_stage1<ST, D, 4>(a, finish, blocks, s);
        case 8: return dispatch_stage1<ST, D, 8>(a, finish, blocks, s);
        default: return hipErrorInvalidValue;
    }
}

template <typename ST, int D>
static const void* stage1_symbol(int gh, bool paged, bool masked) {
    if (masked) {
        switch (gh) {
            case 1: return (const void*)&decode_stage1_kernel<ST, D, 1, kPartial, false, true>;
            case 2: return (const void*)&decode_stage1_kernel<ST, D, 2, kPartial, false, true>;
            case 4: return (const void*)&decode_stage1_kernel<ST, D, 4, kPartial, false, true>;
            case 8: return (const void*)&decode_stage1_kernel<ST, D, 8, kPartial, false, true>;
            default: return nullptr;
        }
    }
    switch (gh) {
        case 1: return paged ? (const void*)&decode_stage1_kernel<ST, D, 1, kPartial, true>
                             : (const void*)&decode_stage1_kernel<ST, D, 1, kPartial, false>;
        case 2: return paged ? (const void*)&decode_stage1_kernel<ST, D, 2, kPartial, true>
                             : (const void*)&decode_stage1_kernel<ST, D, 2, kPartial, false>;
        case 4: return paged ? (const void*)&decode_stage1_kernel<ST, D, 4, kPartial, true>
                             : (const void*)&decode_stage1_kernel<ST, D, 4, kPartial, false>;
        case 8: return paged ? (const void*)&decode_stage1_kernel<ST, D, 8, kPartial, true>
                             : (const void*)&decode_stage1_kernel<ST, D, 8, kPartial, false>;
        default: return nullptr;
    }
}

int decode_stage1_residency(int dtype, int head_dim, int heads_per_wg, bool paged, bool masked) {
    const void* f = nullptr;
    if (dtype == 1) {
        if (head_dim == 64) f = stage1_symbol<BF16, 64>(heads_per_wg, paged, masked);
        if (head_dim == 128) f = stage1_symbol<BF16, 128>(heads_per_wg, paged, masked);
        if (head_dim == 256) f = stage1_symbol<BF16, 256>(heads_per_wg, paged, masked);
    } else {
        if (head_dim == 64) f = stage1_symbol<F16, 64>(heads_per_wg, paged, masked);
        if (head_dim == 128) f = stage1_symbol<F16, 128>(heads_per_wg, paged, masked);
        if (head_dim == 256) f = stage1_symbol<F16, 256>(heads_per_wg, paged, masked);
    }
    int n = 0;
    if (!f || hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, f, 256, 0) != hipSuccess) {
        (void)hipGetLastError();  // no device answered: leave no sticky error behind
        return 0;
    }
    return n;
}

hipError_t launch_decode_stage1(const DecodeArgs& a, int dtype, int head_dim, int heads_per_wg,
                                bool finish, int64_t batch, hipStream_t stream) {
    const int64_t blocks = (int64_t)a.num_splits * batch * a.num_kv_heads * a.head_groups;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (dtype == 1) {
        if (head_dim == 128) return dispatch_stage1_gh<BF16, 128>(a, heads_per_wg, finish, blocks, stream);
        if (head_dim == 64) return dispatch_stage1_gh<BF16, 64>(a, heads_per_wg, finish, blocks, stream);
        if (head_dim == 256) return dispatch_stage1_gh<BF16, 256>(a, heads_per_wg, finish, blocks, stream);
    } else {
        if (head_dim == 128) return dispatch_stage1_gh<F16, 128>(a, heads_per_wg, finish, blocks, stream);
        if (head_dim == 64) return dispatch_stage1_gh<F16, 64>(a, heads_per_wg, finish, blocks, stream);
        if (head_dim == 256) return dispatch_stage1_gh<F16, 256>(a, heads_per_wg, finish, blocks, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_combine(const CombineArgs& a, int dtype, int head_dim, hipStream_t stream) {
    if (a.rows <= 0) return hipSuccess;
    if (a.rows > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)a.rows);
    if (dtype == 1) {
        if (head_dim == 128) hipLaunchKernelGGL((combine_kernel<BF16, 128>), grid, dim3(256), 0, stream, a);
        else if (head_dim == 64) hipLaunchKernelGGL((combine_kernel<BF16, 64>), grid, dim3(256), 0, stream, a);
        else if (head_dim == 256) hipLaunchKernelGGL((combine_kernel<BF16, 256>), grid, dim3(256), 0, stream, a);
        else return hipErrorInvalidValue;
    } else {
        if (head_dim == 128) hipLaunchKernelGGL((combine_kernel<F16, 128>), grid, dim3(256), 0, stream, a);
        else if (head_dim == 64) hipLaunchKernelGGL((combine_kernel<F16, 64>), grid, dim3(256), 0, stream, a);
        else if (head_dim == 256) hipLaunchKernelGGL((combine_kernel<F16, 256>), grid, dim3(256), 0, stream, a);
        else return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace fa
