// fa_decode_mfma.hip -- split-KV decode stage 1 on the matrix cores for
// grouped query heads.
//
// Under GQA (IFA guide 1.1, numKeyValueHeads) the g query heads that share a
// KV head read the same K and V rows.  The vector-ALU stage 1 takes one dot
// product per (row, head) with a 16-lane reduction and an exponential on
// every lane of the row's group, which makes it bound by vector work rather
// than HBM once g reaches 4.  Here the g heads are the rows of a 32-row
// matrix tile instead: S^T = K Q^T and O^T = V^T P^T on
// v_mfma_f32_32x32x16_{bf16,f16} exactly as in the prefill kernel, with the
// rows past g zero (their results are dropped).  A workgroup of NWV waves
// takes one (batch, KV head, chunk) unit; K and V tiles of 32*NWV keys go
// HBM -> LDS with direct buffer loads, double buffered; wave w handles keys
// [32w, 32w+32) of each tile with its own online softmax (running max,
// lazy rescale as in the prefill), and two waves are merged through LDS at
// the end.  Two waves (64-key tiles, 64 KB of LDS at D = 128) suit long
// chunks; one wave (32-key tiles, 32 KB) lets five workgroups share a CU, which keeps
// more tile loads in flight when the chunks are a few tiles long and the
// load latency, not the bandwidth, sets the time.  The partial
// (unnormalised O, max in natural-log units, sum)
// has the layout and meaning of the vector-ALU stage 1 (FlashDecoding
// tutorial, stage 1), so the same combine kernel (stage 2) merges it; a
// one-split plan writes the output and lse in place.
#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"
#include "fa_mfma.h"

namespace fa {

// s_waitcnt immediate (gfx9 encoding) for vmcnt(0) with the other counters free.
constexpr int kWaitVmcnt0 = 0x0F70;

template <typename ST, int D, bool FINISH, bool PAGED, int NWV>
__global__ __launch_bounds__(64 * NWV) __attribute__((amdgpu_waves_per_eu(2))) void decode_mfma_kernel(DecodeArgs a) {
    static_assert(NWV == 1 || NWV == 2, "one or two waves");
    using M = Mfma<ST>;
    using V8 = typename M::V8;
    using E = typename M::E;
    constexpr int BN = 32 * NWV;        // keys per KV tile (32 per wave)
    constexpr int NT = 64 * NWV;        // threads
    constexpr int RB = D * 2;           // bytes per LDS row
    constexpr int TB = BN * RB;         // bytes per K or V tile
    constexpr int CPR = D / 8;          // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;       // rows per wave load
    constexpr int NIW = TB / 1024 / NWV;
    constexpr float kPmax = 256.f;
    static_assert(NIW >= 1, "tile too small");
    __shared__ __attribute__((aligned(1024))) unsigned char sK0[TB];
    __shared__ __attribute__((aligned(1024))) unsigned char sK1[TB];
    __shared__ __attribute__((aligned(1024))) unsigned char sV0[TB];
    __shared__ __attribute__((aligned(1024))) unsigned char sV1[TB];
    __shared__ float s_m[NWV][32], s_l[NWV][32];  // two waves: the merge

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5;
    const int col = lane & 31;

    const int64_t blk = blockIdx.x;
    const int g = a.group;
    int64_t split, b, c0, c1;
    int n2, rg = 0;
    if (a.bal_nwg > 0) {
        // Length-balanced pieces: tstar tiles each, cut at the batch's length.
        int64_t tstar, L;
        if (!bal_find(a.lens, a.batch, a.kv_seq, a.num_kv_heads, a.bal_nwg, blk, &tstar, &b, &n2, &split, &L))
            return;
        c0 = split * tstar * 64;
        c1 = c0 + tstar * 64;
        if (c1 > L) c1 = L;
    } else {
        // With several row groups, the groups of one chunk are dispatched to
        // one XCD (its L2 then serves their shared K/V reads).
        int64_t lb = blk;
        if (a.row_groups > 1) {
            lb = xcd_remap(blk, (int64_t)gridDim.x);
            rg = (int)(lb % a.row_groups);
            lb /= a.row_groups;
        }
        split = lb % a.num_splits;
        const int64_t unit = lb / a.num_splits;
        n2 = (int)(unit % a.num_kv_heads);
        b = unit / a.num_kv_heads;
        int64_t L = a.kv_seq;
        if (a.lens) {
            L = a.lens[b];
            L = L < 0 ? 0 : (L > a.kv_seq ? a.kv_seq : L);
        }
        c0 = split * a.chunk;
        c1 = c0 + a.chunk;
        if (c1 > L) c1 = L;
    }

    // The unit is the same on every lane; stating it keeps the K/V addresses
    // and buffer resources in scalar registers (without it every tile load
    // runs in a loop over the lanes' distinct resources).
    b = uni64(b);
    split = uni64(split);
    c0 = uni64(c0);
    c1 = uni64(c1);
    n2 = __builtin_amdgcn_readfirstlane(n2);
    rg = __builtin_amdgcn_readfirstlane(rg);

    // Tile row col is row r = 32 * rg + col of the KV head's g * Q_S rows,
    // head h = r / Q_S of the group at query position qi = r % Q_S.  Rows at
    // or past the batch's used positions exist (their outputs are written, as
    // empty) but see no key.
    const int QS = (int)a.q_seq;
    const int nrows = g * QS;
    const int used = a.used_q ? min(max(a.used_q[b], 0), QS) : QS;
    int64_t kv_hi = a.kv_seq;  // keys any live row of the batch can see, from the masks
    if (a.mask_mode == 1 && kv_hi > used) kv_hi = used;
    if (a.mask_mode == 3 && kv_hi > (int64_t)used + a.win_right) kv_hi = (int64_t)used + a.win_right;
    if (used == 0) kv_hi = 0;
    kv_hi = uni64(kv_hi);
    if (c1 > kv_hi) c1 = kv_hi;

    // Output row (b, n1, i) of tile row t of this row group, and where its
    // output starts in the q layout.
    auto out_row = [&](int t) __attribute__((always_inline)) {
        const int r = 32 * rg + t;
        return ((b * a.num_heads + (int64_t)n2 * g + r / QS) * a.q_seq + r % QS);
    };
    auto out_elem = [&](int t) __attribute__((always_inline)) {
        const int r = 32 * rg + t;
        return b * a.q_stride_b + ((int64_t)n2 * g + r / QS) * a.q_stride_n + (int64_t)(r % QS) * a.q_stride_s;
    };
    const int tile_rows = min(32, nrows - 32 * rg);  // rows of this row group

    if (c1 <= c0) {
        // A chunk at or past the length (or the masks' reach): its empty
        // partial (or the row defaults of a one-split plan) without touching
        // K or V.
        for (int idx = tid; idx < tile_rows * D; idx += NT) {
            const int h = idx / D;
            const int d = idx % D;
            const int64_t row = out_row(h);
            if constexpr (FINISH) {
                reinterpret_cast<uint16_t*>(a.out)[out_elem(h) + d] = 0;
                if (d == 0 && a.lse) a.lse[row] = kPosInf;
            } else {
                const int64_t slot = row * a.num_splits + split;
                a.o_part[slot * D + d] = 0.f;
                if (d == 0) {
                    a.m_part[slot] = kNegInf;
                    a.l_part[slot] = 0.f;
                }
            }
        }
        return;
    }

    // Q^T as the B operand: lane (col, half) holds head n2*g + col, head-dim
    // elements [16*kk + 8*half, +8).  A negative scale flips the sign bits so
    // the scores are scaled by |scale| * log2(e) > 0.
    const int my_r = 32 * rg + col;
    const bool qexists = col < tile_rows;          // a row of the KV head (written)
    const int my_h = my_r / QS, my_i = my_r % QS;  // its head in the group and query position
    const bool qvalid = qexists && my_i < used;    // it sees keys
    const float c = fabsf(a.scale_log2);
    V8 qreg[D / 16];
    {
        const uint16_t* qp = a.q + b * a.q_stride_b + ((int64_t)n2 * g + my_h) * a.q_stride_n + (int64_t)my_i * a.q_stride_s;
        const uint32_t flip = a.scale_log2 < 0.f ? 0x80008000u : 0u;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            u32x4 w = u32x4{0u, 0u, 0u, 0u};
            if (qvalid && !a.zero_q) w = ld128(qp + kk * 16 + 8 * half);
            w ^= flip;
            qreg[kk] = __builtin_bit_cast(V8, w);
        }
    }
    // Masking beyond the chunk's end: wave-uniform flags.  A row group with
    // rows that see no key masks them on every tile.
    const bool dead_rows = __any(qexists && !qvalid);
    const int mmode = a.mask_mode;
    const uint8_t* mrow = a.mask + b * a.mask_stride[0] + ((int64_t)n2 * g + my_h) * a.mask_stride[1] +
                          (int64_t)my_i * a.mask_stride[2];
    const int64_t mst = a.mask_stride[3];

    f32x16 o[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
    float m_run = kNegInf;  // per head (lane column): reference max, scaled base-2 units
    float tm = kNegInf;     // true running max (the partial reports it)
    float l_half = 0.f;

    // Tile jt holds keys c0 + 64*jt + [0, 64); the buffer resource stops at
    // the chunk's end, so rows past it land as zeros.
    const int64_t row_bytes = a.kv_stride_s * 2;
    const int64_t head_off = PAGED ? (int64_t)n2 * a.kv_stride_n : b * a.kv_stride_b + (int64_t)n2 * a.kv_stride_n;
    const char* kbase = reinterpret_cast<const char*>(a.k + head_off) + (PAGED ? 0 : c0 * row_bytes);
    const char* vbase = reinterpret_cast<const char*>(a.v + head_off) + (PAGED ? 0 : c0 * row_bytes);
    const int64_t nkeys = c1 - c0;
    const int ntiles = (int)((nkeys + BN - 1) / BN);
    // Paged cache: the block ids of the chunk's logical blocks [cb, cb + nblk),
    // clamped into the physical range.  A wave load covers RPI (4 or 8)
    // consecutive rows, and block sizes are multiples of 16, so its rows lie in
    // one block: each wave load takes its own block base.  (Past the chunk's
    // end a load reads nothing -- its byte range is 0 -- whatever block it names.)
    // Two waves stage the ids in LDS; one wave keeps them in a register, lane
    // i holding block i (its chunks span at most kLaneBlocks blocks, which the
    // host plan guarantees), so its LDS stays at the two tile buffers.
    __shared__ int32_t s_blk[(PAGED && NWV == 2) ? kPagedTableLds : 1];
    int32_t lane_blk = 0;
    int64_t cb = 0;
    if constexpr (PAGED) {
        const int bs = a.block_size;
        cb = c0 / bs;
        const int64_t nblk = (c1 - 1) / bs - cb + 1;
        const int32_t* tb = a.block_table + b * a.max_blocks + cb;
        auto clamp_id = [&](int32_t id) { return id < 0 ? 0 : (id >= a.num_blocks ? a.num_blocks - 1 : id); };
        if constexpr (NWV == 1) {
            if (lane < nblk) lane_blk = clamp_id(tb[lane]);
        } else {
            for (int64_t i = tid; i < nblk && i < kPagedTableLds; i += NT) s_blk[i] = clamp_id(tb[i]);
            __syncthreads();
        }
    }
    int voff[NIW];
#pragma unroll
    for (int w = 0; w < NIW; ++w) {
        const int r = RPI * (wave * NIW + w) + lane / CPR;
        const int rr = PAGED ? lane / CPR : r;  // paged: offsets from the wave load's first row
        voff[w] = (int)(rr * row_bytes) + (((lane % CPR) ^ swz<D>(r)) << 4);
    }
    // Paged: a (logical block, row in block) cursor at this wave's next wave
    // load, advanced by additions only (tiles are issued in order): one
    // division here instead of a 64-bit division per wave load.
    int cur_blk = 0, cur_row = 0;
    if constexpr (PAGED) {
        const int64_t t0 = c0 + RPI * (wave * NIW);
        cur_blk = (int)(t0 / a.block_size - cb);
        cur_row = (int)(t0 % a.block_size);
    }
    auto issue_tile = [&](int jt, unsigned char* dK, unsigned char* dV) __attribute__((always_inline)) {
        if constexpr (PAGED) {
            const int bs = a.block_size;
#pragma unroll
            for (int w = 0; w < NIW; ++w) {
                const int I = wave * NIW + w;
                const int64_t t = c0 + (int64_t)jt * BN + RPI * I;  // first key of this wave load
                int64_t rows = c1 - t;
                rows = rows < 0 ? 0 : (rows > RPI ? RPI : rows);
                const int nrec = (int)(rows * row_bytes);
                int32_t id;
                if constexpr (NWV == 1) {
                    id = __builtin_amdgcn_readlane(lane_blk, cur_blk < kLaneBlocks - 1 ? cur_blk : kLaneBlocks - 1);
                } else {
                    const int lb = cur_blk < kPagedTableLds - 1 ? cur_blk : kPagedTableLds - 1;
                    id = __builtin_amdgcn_readfirstlane(s_blk[lb]);
                }
                const int64_t off = ((int64_t)id * a.kv_stride_blk + (int64_t)cur_row * a.kv_stride_s) * 2;
                if constexpr (NWV == 1) {  // as for the contiguous cache below
                    lds_dma16_stream(make_dma_rsrc(kbase + off, nrec), (lds_void*)(dK + I * 1024), voff[w]);
                    lds_dma16_stream(make_dma_rsrc(vbase + off, nrec), (lds_void*)(dV + I * 1024), voff[w]);
                } else {
                    lds_dma16(kbase + off, nrec, (lds_void*)(dK + I * 1024), voff[w]);
                    lds_dma16(vbase + off, nrec, (lds_void*)(dV + I * 1024), voff[w]);
                }
                // Next wave load: RPI rows on (RPI <= 8 < 16 <= bs: at most one
                // block boundary).
                cur_row += RPI;
                if (cur_row >= bs) {
                    cur_row -= bs;
                    ++cur_blk;
                }
            }
            // Two waves: the other wave's 32 rows of the tile lie between this
            // wave's loads of consecutive tiles.
            if constexpr (NWV == 2) {
                cur_row += 32;
                while (cur_row >= bs) {
                    cur_row -= bs;
                    ++cur_blk;
                }
            }
        } else {
            int64_t rows = nkeys - (int64_t)jt * BN;
            rows = rows > BN ? BN : rows;
            const int nrec = (int)(rows * row_bytes);
            const dma_rsrc rk = make_dma_rsrc(kbase + (int64_t)jt * BN * row_bytes, nrec);
            const dma_rsrc rv = make_dma_rsrc(vbase + (int64_t)jt * BN * row_bytes, nrec);
#pragma unroll
            for (int w = 0; w < NIW; ++w) {
                const int I = wave * NIW + w;
                // One wave: loads the compiler does not see (it would wait for
                // them before every LDS read of the step).  Two waves measured
                // faster with the compiler's loads and waits.
                if constexpr (NWV == 1) {
                    lds_dma16_stream(rk, (lds_void*)(dK + I * 1024), voff[w]);
                    lds_dma16_stream(rv, (lds_void*)(dV + I * 1024), voff[w]);
                } else {
                    lds_dma16(kbase + (int64_t)jt * BN * row_bytes, nrec, (lds_void*)(dK + I * 1024), voff[w]);
                    lds_dma16(vbase + (int64_t)jt * BN * row_bytes, nrec, (lds_void*)(dV + I * 1024), voff[w]);
                }
            }
        }
    };

    // LDS read addressing (as in the prefill): K rows 32*wave + col at logical
    // chunk 2*kk + half; V^T through transposing reads of rows
    // 32*wave + 16*ks + {vrow_lo, vrow_hi}.
    const int krow = 32 * wave + col;
    const int ksw = swz<D>(krow);
    const int trG = lane >> 4;
    const int trL = lane & 15;
    const int vrow_lo = 4 * (trG >> 1) + (trL >> 2);
    const int vrow_hi = vrow_lo + 8;
    const int vx = 2 * (trG & 1) + ((trL & 3) >> 1);
    const int vbyte = (trL & 1) * 8;

    // Boolean mask held as whole dwords (4-aligned rows, unit key stride):
    // this lane's four words of a tile (keys 32*wave + 8*q4 + 4*half + [0, 4))
    // are loaded one step ahead, so the wait at the end of each step covers
    // them and the tile's masking never waits on memory.  Words past the
    // chunk are not read.
    const bool mdw = (mmode == 2 && qvalid && a.mask_dword);
    uint32_t mw[4] = {0u, 0u, 0u, 0u};
    auto load_mask_words = [&](int jt) __attribute__((always_inline)) {
        const int64_t kb = c0 + (int64_t)jt * BN + 32 * wave + 4 * half;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int64_t j = kb + 8 * q4;
            mw[q4] = (j < c1) ? *reinterpret_cast<const uint32_t*>(mrow + j) : 0u;
        }
    };

    // The tile loads (inline assembly) are invisible to the compiler's wait
    // placement; the waits below are visible to it and cover its own loads
    // (q, mask words) too, so it places none inside the loop, where a wait on
    // those would also wait for the next tile in flight.
    issue_tile(0, sK0, sV0);
    if (mdw) load_mask_words(0);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();

    auto step = [&](int jt, const unsigned char* Kb, const unsigned char* Vb, unsigned char* nK,
                    unsigned char* nV) __attribute__((always_inline)) {
        // Boolean mask: bit r set when key r of this lane's (row, 16 keys) is
        // masked.  Keys past the chunk are not read.
        uint32_t mbits = 0u;
        if (mdw) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const uint32_t w = mw[q4];
                mbits |= ((w & 0xffu) ? 1u : 0u) << (4 * q4);
                mbits |= ((w & 0xff00u) ? 1u : 0u) << (4 * q4 + 1);
                mbits |= ((w & 0xff0000u) ? 1u : 0u) << (4 * q4 + 2);
                mbits |= ((w & 0xff000000u) ? 1u : 0u) << (4 * q4 + 3);
            }
        }
        if (jt + 1 < ntiles) {
            issue_tile(jt + 1, nK, nV);
            if (mdw) load_mask_words(jt + 1);
        }
        if (mmode == 2 && qvalid && !a.mask_dword) {  // byte loads, in this step
            const int64_t kb = c0 + (int64_t)jt * BN + 32 * wave + 4 * half;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int64_t j = kb + 8 * q4;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (j + e < c1 && mrow[(j + e) * mst] != 0) mbits |= 1u << (4 * q4 + e);
            }
        }
        // S^T: keys 32*wave + [0, 32) of the tile x the 32 head rows.
        // One wave: every K fragment is read before the products, so only the
        // first read's latency is exposed (a one-wave workgroup has no other
        // wave of its own to hide LDS latency); two waves read as they go.
        f32x16 s;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = 0.f;
        if constexpr (NWV == 1) {
            V8 kf[D / 16];
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk)
                kf[kk] = __builtin_bit_cast(
                    V8, *reinterpret_cast<const u32x4*>(Kb + krow * RB + (((2 * kk + half) ^ ksw) << 4)));
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) s = M::mm(kf[kk], qreg[kk], s);
            __builtin_amdgcn_sched_barrier(0);
        } else {
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) {
                const V8 ka = __builtin_bit_cast(
                    V8, *reinterpret_cast<const u32x4*>(Kb + krow * RB + (((2 * kk + half) ^ ksw) << 4)));
                s = M::mm(ka, qreg[kk], s);
            }
        }
        // One wave: the V^T fragments of this wave's keys, read now so their
        // latency passes under the masking and the exponentials.
        V8 vf[2][D / 32];
        auto read_v = [&](int ks, int dt) __attribute__((always_inline)) {
            const int lc = 4 * dt + vx;
            const unsigned char* vb = Vb + (32 * wave + 16 * ks) * RB;
            const int rlo = 32 * wave + 16 * ks + vrow_lo, rhi = rlo + 8;
            const s16x4 lo = lds_read_tr(vb + vrow_lo * RB + ((lc ^ swz<D>(rlo)) << 4) + vbyte);
            const s16x4 hi = lds_read_tr(vb + vrow_hi * RB + ((lc ^ swz<D>(rhi)) << 4) + vbyte);
            return __builtin_bit_cast(V8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        if constexpr (NWV == 1)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
                const int lc = 4 * dt + vx;
                const unsigned char* vb = Vb + (32 * wave + 16 * ks) * RB;
                const int rlo = 32 * wave + 16 * ks + vrow_lo, rhi = rlo + 8;
                const s16x4 lo = lds_read_tr(vb + vrow_lo * RB + ((lc ^ swz<D>(rlo)) << 4) + vbyte);
                const s16x4 hi = lds_read_tr(vb + vrow_hi * RB + ((lc ^ swz<D>(rhi)) << 4) + vbyte);
                vf[ks][dt] = __builtin_bit_cast(V8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        // Register r holds key 32*wave + 8*(r/4) + 4*half + r%4 of the tile.
        const int64_t kt0 = (int64_t)jt * BN + 32 * wave;
        if (kt0 + 32 > nkeys || mmode != 0 || dead_rows) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t key = kt0 + 8 * (r >> 2) + 4 * half + (r & 3);
                const int64_t j = c0 + key;  // absolute key index
                bool ok = key < nkeys && qvalid;
                if (mmode == 1) ok = ok && j <= my_i;
                if (mmode == 3) ok = ok && j >= (int64_t)my_i - a.win_left && j <= (int64_t)my_i + a.win_right;
                if (mmode == 2) ok = ok && ((mbits >> r) & 1u) == 0u;
                s[r] = ok ? s[r] : kNegInf;
            }
        }
        {
            float tmx = kNegInf;
#pragma unroll
            for (int r = 0; r < 16; ++r) tmx = fmaxf(tmx, s[r]);
            tm = fmaxf(tm, fmaxf(tmx, xor32(tmx)) * c);
        }
        V8 pb[2];
        float psum = 0.f;
        auto exps = [&](float nmx) __attribute__((always_inline)) {
            psum = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = fast_exp2(__builtin_fmaf(s[r], c, nmx));
                psum += p;
                pb[r >> 3][r & 7] = (E)p;
            }
        };
        exps((m_run == kNegInf) ? 0.f : -m_run);
        // Lazy rescale, as in the prefill: a half-row sum of at most kPmax
        // shows no score passed the running max by more than 8.
        if (__any(psum > kPmax || (m_run == kNegInf && qvalid))) {
            float tmax = kNegInf;
#pragma unroll
            for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, s[r]);
            tmax = fmaxf(tmax, xor32(tmax)) * c;
            const float mnew = fmaxf(m_run, tmax);
            const float alpha = fast_exp2(m_run - ((mnew == kNegInf) ? 0.f : mnew));
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
            l_half *= alpha;
            m_run = mnew;
            exps((m_run == kNegInf) ? 0.f : -m_run);
        }
        l_half += psum;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
                o[dt] = M::mm(NWV == 1 ? vf[ks][dt] : read_v(ks, dt), pb[ks], o[dt]);
        }
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // the next tile (and mask words) landed
        __syncthreads();
    };
    for (int jt = 0; jt < ntiles; jt += 2) {
        step(jt, sK0, sV0, sK1, sV1);
        if (jt + 1 < ntiles) step(jt + 1, sK1, sV1, sK0, sV0);
    }

    if constexpr (NWV == 1) {
        // Move from the reference max to the true max, as the partial reports
        // the chunk's maximum score; lane (col, half) then holds head col,
        // head-dim elements dt*32 + 8*(r/4) + 4*half + [0, 4).
        float l_run = l_half + xor32(l_half);
        if (tm != kNegInf && tm != m_run) {
            const float f = fast_exp2(m_run - tm);
            l_run *= f;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[dt][r] *= f;
        }
        if (qexists) {
            const int64_t row = out_row(col);
            const bool empty = (tm == kNegInf);
            if constexpr (FINISH) {
                const float inv = empty ? 0.f : 1.f / l_run;
                uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + out_elem(col);
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        const int d = dt * 32 + 8 * q4 + 4 * half;
                        u32x2 w;
                        w[0] = pack2<ST>(o[dt][4 * q4] * inv, o[dt][4 * q4 + 1] * inv);
                        w[1] = pack2<ST>(o[dt][4 * q4 + 2] * inv, o[dt][4 * q4 + 3] * inv);
                        *reinterpret_cast<u32x2*>(op + d) = w;
                    }
                if (half == 0 && a.lse) a.lse[row] = empty ? kPosInf : (tm + log2f(l_run)) * kLn2;
            } else {
                const int64_t slot = row * a.num_splits + split;
                float* op = a.o_part + slot * D;
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        const int d = dt * 32 + 8 * q4 + 4 * half;
                        *reinterpret_cast<f32x4*>(op + d) =
                            f32x4{o[dt][4 * q4], o[dt][4 * q4 + 1], o[dt][4 * q4 + 2], o[dt][4 * q4 + 3]};
                    }
                if (half == 0) {
                    a.m_part[slot] = empty ? kNegInf : tm * kLn2;
                    a.l_part[slot] = l_run;
                }
            }
        }
    } else {
        // Merge the two waves through LDS (the K buffers are free now; wave w
        // writes its [head][D] outputs to sK<w>): per head, M = max of the waves'
        // maxima, A = sum f_w O_w, L = sum f_w l_w with f_w = 2^(m_w - M).
        static_assert(32 * D * 4 == TB, "one wave's outputs fill one K buffer");
        float* s_ow = reinterpret_cast<float*>(wave ? sK1 : sK0);
        const float* s_o0 = reinterpret_cast<const float*>(sK0);
        const float* s_o1 = reinterpret_cast<const float*>(sK1);
        // Move from the reference max to the true max, as the partial reports
        // the chunk's maximum score.
        float l_run = l_half + xor32(l_half);
        if (tm != kNegInf && tm != m_run) {
            const float f = fast_exp2(m_run - tm);
            l_run *= f;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[dt][r] *= f;
        }
        m_run = tm;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int d = dt * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                s_ow[col * D + d] = o[dt][r];
            }
        if (half == 0) {
            s_m[wave][col] = m_run;
            s_l[wave][col] = l_run;
        }
        __syncthreads();
        for (int idx = tid; idx < tile_rows * D; idx += NT) {
            const int h = idx / D;
            const int d = idx % D;
            const float m0 = s_m[0][h], m1 = s_m[1][h];
            const float Mx = fmaxf(m0, m1);
            const float ms = (Mx == kNegInf) ? 0.f : Mx;
            const float f0 = fast_exp2(m0 - ms), f1 = fast_exp2(m1 - ms);
            const float A = __builtin_fmaf(s_o1[h * D + d], f1, s_o0[h * D + d] * f0);
            const float Lt = __builtin_fmaf(s_l[1][h], f1, s_l[0][h] * f0);
            const int64_t row = out_row(h);
            if constexpr (FINISH) {
                const bool empty = (Mx == kNegInf);
                reinterpret_cast<uint16_t*>(a.out)[out_elem(h) + d] = to_bits<ST>(empty ? 0.f : A / Lt);
                if (d == 0 && a.lse) a.lse[row] = empty ? kPosInf : (Mx + log2f(Lt)) * kLn2;
            } else {
                const int64_t slot = row * a.num_splits + split;
                a.o_part[slot * D + d] = A;
                if (d == 0) {
                    a.m_part[slot] = (Mx == kNegInf) ? kNegInf : Mx * kLn2;
                    a.l_part[slot] = Lt;
                }
            }
        }
    }
}

template <typename ST, int D, int NWV>
static const void* mfma_symbol(bool paged) {
    return paged ? (const void*)&decode_mfma_kernel<ST, D, false, true, NWV>
                 : (const void*)&decode_mfma_kernel<ST, D, false, false, NWV>;
}

template <int NWV>
static const void* mfma_symbol_for(int dtype, int head_dim, bool paged) {
    if (head_dim == 64) return dtype == 1 ? mfma_symbol<BF16, 64, NWV>(paged) : mfma_symbol<F16, 64, NWV>(paged);
    if (head_dim == 128) return dtype == 1 ? mfma_symbol<BF16, 128, NWV>(paged) : mfma_symbol<F16, 128, NWV>(paged);
    return nullptr;
}

int decode_mfma_residency(int dtype, int head_dim, bool paged, int waves) {
    const void* f = waves == 1 ? mfma_symbol_for<1>(dtype, head_dim, paged) : mfma_symbol_for<2>(dtype, head_dim, paged);
    int n = 0;
    if (!f || hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, f, 64 * waves, 0) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    return n;
}

template <typename ST, int D, int NWV>
static hipError_t dispatch_mfma(const DecodeArgs& a, bool finish, int64_t blocks, hipStream_t s) {
    const dim3 grid((unsigned)blocks), block(64 * NWV);
    if (a.block_table) {
        if (finish)
            hipLaunchKernelGGL((decode_mfma_kernel<ST, D, true, true, NWV>), grid, block, 0, s, a);
        else
            hipLaunchKernelGGL((decode_mfma_kernel<ST, D, false, true, NWV>), grid, block, 0, s, a);
    } else {
        if (finish)
            hipLaunchKernelGGL((decode_mfma_kernel<ST, D, true, false, NWV>), grid, block, 0, s, a);
        else
            hipLaunchKernelGGL((decode_mfma_kernel<ST, D, false, false, NWV>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

template <typename ST, int D>
static hipError_t dispatch_mfma_waves(const DecodeArgs& a, bool finish, int waves, int64_t blocks, hipStream_t s) {
    return waves == 1 ? dispatch_mfma<ST, D, 1>(a, finish, blocks, s) : dispatch_mfma<ST, D, 2>(a, finish, blocks, s);
}

hipError_t launch_decode_mfma(const DecodeArgs& a, int dtype, int head_dim, bool finish, int waves, int64_t batch,
                              hipStream_t stream) {
    if (a.group < 1 || a.group > 32) return hipErrorInvalidValue;
    if (waves != 1 && waves != 2) return hipErrorInvalidValue;
    if (a.block_table && (a.block_size < 16 || a.block_size % 16 != 0)) return hipErrorInvalidValue;
    if (a.bal_nwg > 0 && (finish || !a.lens || a.batch != batch)) return hipErrorInvalidValue;
    if (a.row_groups < 1 || a.row_groups > 16 || a.group * a.q_seq > 32 * a.row_groups) return hipErrorInvalidValue;
    if (a.bal_nwg > 0 && (a.row_groups != 1 || a.q_seq != 1 || a.mask_mode != 0 || a.used_q))
        return hipErrorInvalidValue;
    const int64_t blocks = a.bal_nwg > 0 ? (int64_t)a.bal_nwg + batch * a.num_kv_heads
                                         : (int64_t)a.num_splits * batch * a.num_kv_heads * a.row_groups;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (dtype == 1) {
        if (head_dim == 128) return dispatch_mfma_waves<BF16, 128>(a, finish, waves, blocks, stream);
        if (head_dim == 64) return dispatch_mfma_waves<BF16, 64>(a, finish, waves, blocks, stream);
    } else {
        if (head_dim == 128) return dispatch_mfma_waves<F16, 128>(a, finish, waves, blocks, stream);
        if (head_dim == 64) return dispatch_mfma_waves<F16, 64>(a, finish, waves, blocks, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace fa
