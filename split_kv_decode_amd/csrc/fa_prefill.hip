// fa_prefill.hip -- tiled attention forward on gfx950 matrix cores.
//
// For one (batch, query head, 128-row query tile) a workgroup of four waves
// walks the KV sequence in tiles of 64 keys: S = scale*QK^T on MFMA, masking,
// an online softmax (running max m, running sum l, rescale of the output by
// exp(m_old - m_new), as in the FlashSoftmax flow of the IFA guide, section
// 8.1), O += P V on MFMA, and the division by l deferred to the epilogue.  The
// score matrix never leaves registers (FlashAttn operator guide, function
// description: O(tile) memory instead of O(Q_S x KV_S)).
//
// Matrix-core layout.  Each wave owns 32 query rows.  The kernel computes the
// transposed products S^T = K Q^T and O^T = V^T P^T with
// v_mfma_f32_32x32x16_{bf16,f16}: in the 32x32 accumulator a lane holds one
// column (= one query row) and 16 rows (= keys), which is exactly the lane
// layout the B operand of the next MFMA wants for P^T, so P goes from the
// score accumulators to the PV instruction without touching LDS.  The row
// max/sum of the softmax is an in-lane reduction plus one exchange between the
// two half-waves (v_permlane32_swap).  Q stays in registers for the whole KV
// loop.
//
// Memory path.  K and V tiles go from HBM straight into LDS with buffer loads
// (no staging registers), double buffered so the next tile is in flight while
// the current one is consumed; the buffer range check returns zeros for rows
// at or past the batch's length, whatever the cache holds there.  LDS rows are
// unpadded and 16-byte chunks are XOR-swizzled so that both read patterns --
// 16 rows at one chunk for K, and the transposing ds_read_b64_tr_b16 reads
// that build V^T operands -- are free of bank conflicts.
//
// Masks.  MASK 0 none; 1 causal from indices (tiles past the diagonal are
// not visited); 2 a boolean tensor read element by element; 3 a boolean
// tensor with contiguous key rows, staged through LDS with the K/V tiles (a
// wave skips a tile its rows mask entirely, and the element tests of a tile
// that masks none of its rows; given a per-tile summary of the mask, the
// workgroup visits only the tiles between the first and the last one with a
// visible key and loads neither tiles with none nor the mask of tiles that
// mask nothing);
// 4 the window band of the FlashAttn developer guide (1.5, mode 4): only the
// KV tiles that intersect the band of the query tile are visited, and a wave
// skips tiles outside the band of its 32 rows.
//
// Softmax.  Exponentials are taken against the running max before the tile's
// max is known, and the output is rescaled only when a row max grows by more
// than 2^8 (wave-uniform test, decided from the sum of the exponentials, so
// the tile max itself is computed only on that rare path); the vector work
// per tile is about one FMA, one exp, one add and half a convert per score.
#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"
#include "fa_mfma.h"

namespace fa {


// D = 256 holds 64 + 128 registers of Q and O per lane, so it runs one
// workgroup per CU with the accumulators in the AGPR half of the file.
// O *= alpha on the rare rescale path.  At D = 256, O lives in the
// accumulation registers (AGPRs) of the products; scaled there in place it
// needs no vector-register copy, which the compiler otherwise made at the top
// of every KV step whether or not this path ran.  Wait states: the last
// product that wrote O is many products back, and each write is followed by
// the two that a product reading it needs.
template <int D>
__device__ __forceinline__ void scale_acc(f32x16 (&o)[D / 32], float alpha) {
    if constexpr (D == 256) {
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" ::: "memory");
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float t;
                asm volatile(
                    "v_accvgpr_read_b32 %1, %0\n\t"
                    "v_mul_f32 %1, %1, %2\n\t"
                    "v_accvgpr_write_b32 %0, %1\n\t"
                    "s_nop 2"
                    : "+a"(o[dt][r]), "=&v"(t)
                    : "v"(alpha));
            }
    } else {
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
    }
}

template <typename ST, int D, int MASK>
__global__ __launch_bounds__(256, (D == 256) ? 1 : 2) void prefill_kernel(PrefillArgs a) {
    using M = Mfma<ST>;
    using V8 = typename M::V8;
    using E = typename M::E;
    constexpr int BM = 128;             // query rows per workgroup (32 per wave)
    constexpr int BN = 64;              // keys per KV tile
    constexpr int RB = D * 2;           // bytes per LDS row (unpadded)
    constexpr int TB = BN * RB;         // bytes per K or V tile
    constexpr int CPR = D / 8;          // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;       // rows per direct-to-LDS wave load
    constexpr int NIW = TB / 1024 / 4;  // wave loads per wave per tile (K, and again V)
    constexpr float kPmax = 256.f;      // rescale only when an exponential could exceed 2^8
    static_assert(BM == kMaskRowsPerTile && BN == kMaskKeysPerTile, "mask summary tiles");
    __shared__ __attribute__((aligned(1024))) unsigned char sK0[TB];
    __shared__ __attribute__((aligned(1024))) unsigned char sK1[TB];
    __shared__ __attribute__((aligned(1024))) unsigned char sV0[TB];
    __shared__ __attribute__((aligned(1024))) unsigned char sV1[TB];
    // MASK 3: the boolean mask tile (128 query rows x 64 keys, one byte each),
    // chunk-major: 16-byte chunk c of row r at (c*128 + r)*16.
    constexpr int MT = (MASK == 3) ? BM * BN : 16;
    __shared__ __attribute__((aligned(1024))) unsigned char sM0[MT];
    __shared__ __attribute__((aligned(1024))) unsigned char sM1[MT];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: LDS DMA bases stay in SGPRs
    const int half = lane >> 5;
    const int col = lane & 31;

    int qt, n1;
    int64_t b, L;
    int64_t q_used = a.q_seq, q_full = a.q_seq;  // query rows computed / written
    int64_t q_off, kv_off;                       // element offsets of (b) in q/out and k/v
    int64_t lse_row0, lse_step;                  // lse index of (n1, row i) = lse_row0 + i * lse_step
    if (a.work) {
        // Packed layout: block 8k + x (dispatched to XCD x) takes head k % N of
        // work item 8*(k / N) + x, so the heaviest items spread over all XCDs
        // and the heads of one item (which share K/V under GQA) share an L2.
        const int x = (int)(blockIdx.x & 7);
        const int64_t kk = blockIdx.x >> 3;
        const int64_t item = (kk / a.num_heads) * 8 + x;
        n1 = (int)(kk % a.num_heads);
        if (item >= a.work_items) return;
        const int32_t wb = a.work[2 * item];
        if (wb < 0) return;
        b = wb;
        qt = a.work[2 * item + 1];
        const SeqGeom sg = seq_geometry(a.cu_q, a.cu_kv, a.used_q, a.lens, b, a.batch, a.q_seq, a.kv_seq);
        q_used = sg.q_used;
        q_full = sg.q_full;
        L = sg.kv_len;
        q_off = sg.q0 * a.q_stride_s;
        kv_off = sg.k0 * a.kv_stride_s;
        lse_row0 = sg.q0 * a.num_heads + n1;
        lse_step = a.num_heads;
    } else {
        const int64_t total = (int64_t)gridDim.x;
        int64_t bh;
        if (MASK == 1 || MASK == 3 || (MASK == 4 && a.win_left >= a.win_right)) {
            // Causal costs grow with the query tile, and so do those of a
            // window that reaches further back than forward (its first tiles
            // are cut at key 0): dispatch every head's tile of one rank before
            // the next lighter rank (longest first over the whole grid, so no
            // heavy tile starts near the end); the heads of a rank keep their
            // XCD, as in the order below.
            const int64_t heads = total / a.q_tiles;
            qt = a.q_tiles - 1 - (int)(blockIdx.x / heads);
            bh = xcd_remap(blockIdx.x % heads, heads);
        } else {
            const int64_t work = xcd_remap(blockIdx.x, total);
            qt = (int)(work % a.q_tiles);
            bh = work / a.q_tiles;
        }
        n1 = (int)(bh % a.num_heads);
        b = bh / a.num_heads;
        L = a.kv_seq;
        if (a.lens) {
            L = a.lens[b];
            L = L < 0 ? 0 : (L > a.kv_seq ? a.kv_seq : L);
        }
        q_off = b * a.q_stride_b;
        kv_off = b * a.kv_stride_b;
        lse_row0 = (b * a.num_heads + n1) * a.q_seq;
        lse_step = 1;
        if (a.used_q) {  // rows at or past the batch's used positions: written as 0 / +inf
            const int64_t u = a.used_q[b];
            q_used = u < 0 ? 0 : (u > a.q_seq ? a.q_seq : u);
        }
    }
    const int n2 = n1 / a.group;

    const int64_t i0 = (int64_t)qt * BM;
    const int64_t wrow0 = i0 + 32 * wave;  // first query row of this wave
    const int64_t qrow = wrow0 + col;
    const bool qvalid = qrow < q_used;

    // Q as the B operand of S^T = K Q^T: lane (col, half) holds row qrow,
    // head-dim elements [16*kk + 8*half, +8).  A negative scale is folded in
    // by flipping the sign bits, so scores are scaled by |scale| * log2(e) > 0
    // and the row max can be taken before scaling.
    V8 qreg[D / 16];
    {
        const uint16_t* qp = a.q + q_off + (int64_t)n1 * a.q_stride_n + qrow * a.q_stride_s;
        const uint32_t flip = a.negate_q ? 0x80008000u : 0u;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            u32x4 w = u32x4{0u, 0u, 0u, 0u};
            if (qvalid && !a.zero_q) w = ld128(qp + kk * 16 + 8 * half);  // zero_q: scale 0
            w ^= flip;
            qreg[kk] = __builtin_bit_cast(V8, w);
        }
    }
    const float c = a.scale_log2;

    // KV tiles [jt0, ntiles) can hold visible keys for this query tile: causal
    // stops at the tile's last row, a window spans from the first row's left
    // edge to the last row's right edge.
    int64_t kv_end = L;
    if (MASK == 1 && kv_end > i0 + BM) kv_end = i0 + BM;  // keys beyond the tile's last row
    int jt0 = 0;
    if (MASK == 4) {
        const int64_t i_last = (i0 + BM < q_used ? i0 + BM : q_used) - 1;
        if (kv_end > i_last + a.win_right + 1) kv_end = i_last + a.win_right + 1;
        const int64_t key_lo = i0 - a.win_left;
        if (key_lo > 0) jt0 = (int)(key_lo / BN);
    }
    int ntiles = (int)((kv_end + BN - 1) / BN);
    if (i0 >= q_used) ntiles = jt0;  // no row of the tile is used: outputs only

    // MASK 3 with a summary of the mask: the row of tile classes of this
    // query tile (two bits per KV tile: some key visible, some key masked).
    // Lane l keeps word l, KV tiles 16l .. 16l+15; the first and the last
    // tile with a visible key bound the loop.  Tiles past the 64 words the
    // lanes keep count as partly masked.
    const bool summary = (MASK == 3) && a.mask_cls != nullptr;
    uint32_t cls_word = 0xffffffffu;
    if (MASK == 3 && summary) {
        const int64_t sn = a.mask_stride[1] ? a.num_heads : 1;
        const int64_t slice = (a.mask_stride[0] ? b : 0) * sn + (a.mask_stride[1] ? n1 : 0);
        const uint32_t* crow = a.mask_cls + (slice * a.q_tiles + qt) * a.cls_words;
        int first = 0x7fffffff, last = -1;
        for (int w = lane; w < a.cls_words; w += 64) {
            const uint32_t x = crow[w];
            if (w == lane) cls_word = x;
            const uint32_t live = x & 0x55555555u;
            if (live) {
                first = min(first, 16 * w + (__builtin_ctz(live) >> 1));
                last = max(last, 16 * w + ((31 - __builtin_clz(live)) >> 1));
            }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            first = min(first, __shfl_xor(first, off, 64));
            last = max(last, __shfl_xor(last, off, 64));
        }
        first = __builtin_amdgcn_readfirstlane(first);
        last = __builtin_amdgcn_readfirstlane(last);
        if (first > jt0) jt0 = first;
        if (last + 1 < ntiles) ntiles = last + 1;
    }
    auto tile_cls = [&](int jt) __attribute__((always_inline)) -> uint32_t {
        if (!summary || jt >= 64 * 16) return 3u;
        return (__builtin_amdgcn_readlane(cls_word, jt >> 4) >> (2 * (jt & 15))) & 3u;
    };

    f32x16 o[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
    float m_run = kNegInf;  // per query row, scaled base-2 units (same in both halves)
    float l_half = 0.f;     // this half-wave's share of the row sum

    // Direct-to-LDS tile loads.  Wave load I of a tile fills LDS bytes
    // [1024*I, +1024): lane i writes 16 bytes at 16*i, i.e. row RPI*I + i/CPR,
    // physical chunk i%CPR, which holds logical chunk (i%CPR) ^ swz(row).  The
    // buffer resource of a tile covers only its rows below the length.
    const int64_t row_bytes = a.kv_stride_s * 2;
    const char* kbase = reinterpret_cast<const char*>(a.k + kv_off + (int64_t)n2 * a.kv_stride_n);
    const char* vbase = reinterpret_cast<const char*>(a.v + kv_off + (int64_t)n2 * a.kv_stride_n);
    int voff[NIW];
#pragma unroll
    for (int w = 0; w < NIW; ++w) {
        const int r = RPI * (wave * NIW + w) + lane / CPR;
        voff[w] = (int)(r * row_bytes) + (((lane % CPR) ^ swz<D>(r)) << 4);
    }
    // MASK 3 mask tile: wave w loads chunk w (keys 16*w .. 16*w+15) of all
    // 128 rows, 64 rows per wave load.  The resource stops at the last valid
    // row's last key, so nothing past the mask tensor is read.
    const char* mbase = reinterpret_cast<const char*>(a.mask) + b * a.mask_stride[0] +
                        (int64_t)n1 * a.mask_stride[1] + i0 * a.mask_stride[2];
    int moff[2] = {0, 0};
    int mrec_rows = 0;
    if (MASK == 3) {
#pragma unroll
        for (int w = 0; w < 2; ++w) moff[w] = (int)((w * 64 + lane) * a.mask_stride[2]) + wave * 16;
        int64_t rv = q_used - i0;
        rv = rv > BM ? BM : rv;
        mrec_rows = (int)((rv - 1) * a.mask_stride[2]);
    }
    auto issue_tile = [&](int jt, unsigned char* dK, unsigned char* dV, unsigned char* dM)
                          __attribute__((always_inline)) {
        const uint32_t cls = (MASK == 3) ? tile_cls(jt) : 3u;
        if (MASK == 3 && !(cls & 1u)) return;  // no visible key: nothing to load
        const int64_t j0 = (int64_t)jt * BN;
        int64_t rows = L - j0;
        rows = rows < 0 ? 0 : (rows > BN ? BN : rows);
        const int nrec = (int)(rows * row_bytes);
        const char* kt = kbase + j0 * row_bytes;
        const char* vt = vbase + j0 * row_bytes;
        const dma_rsrc rk = make_dma_rsrc(kt, nrec), rv = make_dma_rsrc(vt, nrec);
#pragma unroll
        for (int w = 0; w < NIW; ++w) {
            const int I = wave * NIW + w;
            lds_dma16_unordered(rk, (lds_void*)(dK + I * 1024), voff[w]);
            lds_dma16_unordered(rv, (lds_void*)(dV + I * 1024), voff[w]);
        }
        if (MASK == 3 && (cls & 2u)) {
            int64_t keys = a.kv_seq - j0;
            keys = keys > BN ? BN : keys;
            const int mrec = mrec_rows + (int)keys;
            const dma_rsrc rm = make_dma_rsrc(mbase + j0, mrec);
#pragma unroll
            for (int w = 0; w < 2; ++w) lds_dma16_unordered(rm, (lds_void*)(dM + (2 * wave + w) * 1024), moff[w]);
        }
    };

    // Per-lane LDS read addresses.  K (A operand of S^T = K Q^T): rows col and
    // 32+col, logical chunk 2*kk+half.  V (transposing reads, see lds_read_tr):
    // 16-lane group G = lane/16 serves head-dim columns 16*(G&1) + [0,16) of a
    // 32-column tile and key slots 4*(G>>1) + [0,4); its source lane Ls =
    // lane%16 addresses key row Ls/4 of those four (+8 for the second read),
    // logical chunk 4*dt + 2*(G&1) + (Ls&3)/2, byte (Ls&1)*8 of it.
    const int krow0 = col, krow1 = 32 + col;
    const int ks0 = swz<D>(krow0), ks1 = swz<D>(krow1);
    const int trG = lane >> 4;
    const int trL = lane & 15;
    const int vrow_lo = 4 * (trG >> 1) + (trL >> 2);
    const int vrow_hi = vrow_lo + 8;
    const int vs_lo = swz<D>(vrow_lo), vs_hi = swz<D>(vrow_hi);
    const int vx = 2 * (trG & 1) + ((trL & 3) >> 1);
    const int vbyte = (trL & 1) * 8;

    if (ntiles > jt0) issue_tile(jt0, sK0, sV0, sM0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // One KV tile: its K/V are in (Kb, Vb); the next tile is loaded into
    // (nK, nV) meanwhile.  The loop below is unrolled by two so every LDS
    // access names a fixed buffer (which also lets the compiler see that the
    // tile being read is not the one the in-flight loads write).
    auto step = [&](int jt, const unsigned char* Kb, const unsigned char* Vb, const unsigned char* Mb,
                    unsigned char* nK, unsigned char* nV, unsigned char* nM) __attribute__((always_inline)) {
        const int64_t j0 = (int64_t)jt * BN;
        if (jt + 1 < ntiles) issue_tile(jt + 1, nK, nV, nM);

        // MASK 3: this lane's 32 mask bytes -- word (tt, g) holds keys
        // 32*tt + 8*g + 4*half + [0,4) of row 32*wave + col -- and a
        // wave-uniform skip of tiles the mask excludes entirely for its rows.
        uint32_t mw[2][4];
        bool mask_clear = false;  // MASK 3: no key of this tile is masked for any row of the wave
        // With a summary, class 1 (no key masked) loaded no mask tile and
        // needs no tests; a tile with no visible key (bit 0 clear) loaded
        // nothing and is skipped by the test below whatever the LDS holds.
        const uint32_t cls = (MASK == 3) ? tile_cls(jt) : 3u;
        if (MASK == 3 && cls == 1u) mask_clear = true;
        if (MASK == 3 && cls != 1u) {
            // zero_bytes gathers the top bit of every zero (visible) byte of
            // the lane's 32 keys, any_set every masked bit; bitwise so the
            // tests stay branch-free.
            uint32_t zero_bytes = 0u, any_set = 0u;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int ch = 2 * tt + (g >> 1);
                    const uint32_t w = *reinterpret_cast<const uint32_t*>(
                        Mb + (ch * BM + 32 * wave + col) * 16 + 8 * (g & 1) + 4 * half);
                    zero_bytes |= (w - 0x01010101u) & ~w & 0x80808080u;
                    any_set |= w;
                }
            }
            const bool lane_all = !qvalid | (j0 >= L) | !(cls & 1u) | (zero_bytes == 0u);
            mask_clear = __all(any_set == 0u);
            if (__all(lane_all)) {
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                __syncthreads();
                return;
            }
        }
        if (MASK == 3) asm volatile("" ::: "memory");  // re-read the words after the QK MFMAs instead of holding them
        // MASK 4: a tile wholly left or right of the band of every row of
        // this wave is skipped (wave-uniform) at D <= 128; at D = 256 the
        // second exit from the step costs more registers than the register
        // file holds, and the tile runs fully masked instead.
        if (MASK == 4 && D <= 128) {
            if (j0 + BN - 1 < wrow0 - a.win_left || j0 > wrow0 + 31 + a.win_right) {
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                __syncthreads();
                return;
            }
        }

        // S^T tiles: keys [j0 + 32*tt, +32) x the wave's 32 query rows (raw
        // q.k); the two accumulation chains are interleaved.
        f32x16 s[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[tt][r] = 0.f;
        // K fragments read PF steps ahead of their products (a ring of
        // PF + 1 register pairs), the order pinned with scheduling barriers.
        constexpr int PF = (D == 256) ? 1 : 2;
        auto kread = [&](int kk, V8* dst) __attribute__((always_inline)) {
            dst[0] = __builtin_bit_cast(
                V8, *reinterpret_cast<const u32x4*>(Kb + krow0 * RB + (((2 * kk + half) ^ ks0) << 4)));
            dst[1] = __builtin_bit_cast(
                V8, *reinterpret_cast<const u32x4*>(Kb + krow1 * RB + (((2 * kk + half) ^ ks1) << 4)));
        };
        V8 kring[PF + 1][2];
#pragma unroll
        for (int p = 0; p < PF; ++p) kread(p, kring[p]);
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            if (kk + PF < D / 16) kread(kk + PF, kring[(kk + PF) % (PF + 1)]);
            __builtin_amdgcn_sched_barrier(0);
            s[0] = M::mm(kring[kk % (PF + 1)][0], qreg[kk], s[0]);
            s[1] = M::mm(kring[kk % (PF + 1)][1], qreg[kk], s[1]);
            __builtin_amdgcn_sched_barrier(0);
        }

        // Masking is needed only on tiles that cross the length, the causal
        // diagonal of this wave's rows, or under a boolean mask.  Accumulator
        // register r of tile tt holds key j0 + 32*tt + 8*(r/4) + 4*half + r%4.
        const bool need_mask = (j0 + BN > L) || (MASK == 1 && j0 + BN - 1 > wrow0) || (MASK == 2) ||
                               (MASK == 3 && !mask_clear) ||
                               (MASK == 4 && (j0 < wrow0 + 31 - a.win_left || j0 + BN - 1 > wrow0 + a.win_right));
        // MASK 3: the lane's mask words, read whatever the class (a tile that
        // masks nothing left stale bytes here, which mask_clear overrides).
        if (MASK == 3) {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    mw[tt][g] = *reinterpret_cast<const uint32_t*>(
                        Mb + ((2 * tt + (g >> 1)) * BM + 32 * wave + col) * 16 + 8 * (g & 1) + 4 * half);
        }
        if (need_mask) {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t tok = j0 + tt * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                    bool ok = tok < L;
                    if (MASK == 1) ok = ok && tok <= qrow;
                    if (MASK == 2)
                        ok = ok && qvalid &&
                             a.mask[b * a.mask_stride[0] + (int64_t)n1 * a.mask_stride[1] +
                                    qrow * a.mask_stride[2] + tok * a.mask_stride[3]] == 0;
                    if (MASK == 3)
                        ok = ok & qvalid & (mask_clear | (((mw[tt][r >> 2] >> (8 * (r & 3))) & 0xffu) == 0u));
                    if (MASK == 4) {
                        const int dj = (int)(tok - qrow);
                        ok = ok && dj >= -a.win_left && dj <= a.win_right;
                    }
                    s[tt][r] = ok ? s[tt][r] : kNegInf;
                }
            }
        }

        // P^T as the B operand of O^T = V^T P^T.  K-step ks covers keys
        // [16*ks, +16) of the tile; slot e of half h is key 4h+e (e<4) or
        // 8+4h+(e-4) -- the order the accumulator already holds them in.
        // Exponentials are taken against the running max; in the rare case a
        // row max grew by more than 8 they are recomputed after the rescale,
        // so every exponential stays below kPmax = 2^8.
        V8 pb[4];
        float psum = 0.f;
        auto exps = [&](float nmx) __attribute__((always_inline)) {
            psum = 0.f;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = fast_exp2(__builtin_fmaf(s[tt][r], c, nmx));
                    psum += p;
                    pb[tt * 2 + (r >> 3)][r & 7] = (E)p;
                }
            }
        };
        exps((m_run == kNegInf) ? 0.f : -m_run);
        // Every p >= 0, so a half-row sum of at most kPmax proves no score
        // exceeded the running max by more than 8: the tile max is needed
        // only on the rare path that moves the max (or while a row of the
        // query has seen no valid key yet, so an empty row keeps m = -inf;
        // rows past the query length never trigger it).
        if (__any(psum > kPmax || (m_run == kNegInf && qvalid))) {
            float tmax = kNegInf;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, s[tt][r]);
            tmax = fmaxf(tmax, xor32(tmax)) * c;
            const float mnew = fmaxf(m_run, tmax);
            const float alpha = fast_exp2(m_run - ((mnew == kNegInf) ? 0.f : mnew));
            scale_acc<D>(o, alpha);
            l_half *= alpha;
            m_run = mnew;
            exps((m_run == kNegInf) ? 0.f : -m_run);
        }
        l_half += psum;

#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
                // A operand V^T: lane (col, half) holds head-dim row 32*dt+col
                // at the key slots of pb[ks]; the two transposing reads give
                // slots 0..3 (keys 4h+[0,4)) and 4..7 (keys 8+4h+[0,4)).
                const int lc = 4 * dt + vx;
                const unsigned char* vb = Vb + ks * 16 * RB;
                const s16x4 lo = lds_read_tr(vb + vrow_lo * RB + ((lc ^ vs_lo) << 4) + vbyte);
                const s16x4 hi = lds_read_tr(vb + vrow_hi * RB + ((lc ^ vs_hi) << 4) + vbyte);
                const V8 va = __builtin_bit_cast(V8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                o[dt] = M::mm(va, pb[ks], o[dt]);
            }
            if constexpr (D == 256) asm volatile("" ::: "memory");
        }

        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's loads of the next tile landed
        __syncthreads();  // ... and everyone else's; this tile is consumed
    };
    for (int jt = jt0; jt < ntiles; jt += 2) {
        step(jt, sK0, sV0, sM0, sK1, sV1, sM1);
        if (jt + 1 < ntiles) step(jt + 1, sK1, sV1, sM1, sK0, sV0, sM0);
    }

    // Epilogue: divide by l, RowInvalid defaults, store in the q layout.  Rows
    // a packed sequence owns but does not use get the initial 0 / +inf.  At
    // D = 256 under a window or staged mask the row is taken again from the
    // lane id, so no per-lane address computed for the q load stays live
    // across the loop (those instantiations otherwise spill it).
    const float l_run = l_half + xor32(l_half);
    constexpr bool kRowFromLane = D == 256 && (MASK == 3 || MASK == 4);
    const int64_t qrow_e = kRowFromLane ? wrow0 + (int)(__lane_id() & 31) : qrow;
    if (qrow_e < q_full) {
        const bool empty = !(qrow_e < q_used) || (m_run == kNegInf);
        const float inv = empty ? 0.f : 1.f / l_run;
        uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + q_off + (int64_t)n1 * a.q_stride_n +
                       qrow_e * a.q_stride_s;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
                const int d0 = dt * 32 + 8 * a4 + 4 * half;
                float x[4];
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) x[cc] = empty ? 0.f : o[dt][4 * a4 + cc] * inv;
                u32x2 w;
                w[0] = pack2<ST>(x[0], x[1]);
                w[1] = pack2<ST>(x[2], x[3]);
                *reinterpret_cast<u32x2*>(op + d0) = w;
            }
        }
        if (half == 0 && a.lse) a.lse[lse_row0 + qrow_e * lse_step] = empty ? kPosInf : (m_run + log2f(l_run)) * kLn2;
    }
}

// Interleaved prefill, used at D = 128 for every mask kind (a boolean tensor
// read element by element excepted, unless its key rows are runs of 4-byte
// aligned words) and for the packed layout: one workgroup of 8 waves per CU,
// 256 query rows (32 per wave), each 64-key K/V tile loaded into LDS once for
// all 8 waves.  Every wave runs the same software-pipelined
// schedule and issues its own matrix and vector work interleaved.  Slot j
// holds K(j) and V(j-1); a wave spends it in two stages:
//   A: the 16 products of S(j) = K(j) Q^T, each pair preceded by two
//      exponentials of the second half (keys 32..63) of tile j-1;
//   B: the 16 products of O += V(j-1)^T P(j-1), each preceded by one
//      exponential of the first half (keys 0..31) of tile j.
// The two waves a SIMD holds then both feed its matrix core between their
// vector instructions.  (A probe of schedules on gfx950 measured the matrix
// core 93 % busy this way, against 82 % when one wave of a SIMD issues only
// products and the other only vector work, which is how an earlier ping-pong
// form of this kernel was arranged; this kernel measured 3-4 % faster than
// it.)  Within each step the order -- LDS fragment reads, vector work,
// products -- is pinned with scheduling barriers, so a read's latency passes
// under the vector work.  Each half-tile checks its own exponential sum for
// the lazy rescale (a half-row sum of at most 2^8 proves no exponential of
// the half exceeded 2^8); the rare rescale takes the maximum over what is
// needed and recomputes what was taken against the old maximum.  K(j+1) is
// loaded at the start of slot j and V(j) after stage A, with every scalar of
// the load worked out beforehand; one barrier per slot releases the buffers.
template <int D>
constexpr int il_waves() { return D == 256 ? 4 : 8; }

template <typename ST, int D, int MASK, bool PERSIST, bool PACKED = false>
__global__ __launch_bounds__(64 * il_waves<D>(), 1) void prefill_il_kernel(PrefillArgs a) {
    static_assert(MASK >= 0 && MASK <= 4, "mask kind");
    static_assert(D == 128 || D == 256, "head dim");
    static_assert(!PERSIST || MASK == 0 || MASK == 1 || MASK == 4, "persistent launch: no mask, causal or window");
    static_assert(!PACKED || PERSIST, "PACKED: the persistent kernel of the packed layout");
    using M = Mfma<ST>;
    using V8 = typename M::V8;
    using E = typename M::E;
    // D = 128: 8 waves, two per SIMD.  D = 256: Q (64 registers) and O (128)
    // per lane leave room for one wave per SIMD, so 4 waves and 128 rows,
    // with O in the accumulation registers.
    constexpr int NWV = il_waves<D>();  // waves
    constexpr int BN = 64;              // keys per KV tile
    constexpr int RB = D * 2;
    constexpr int TB = BN * RB;
    constexpr int CPR = D / 8;
    constexpr int RPI = 64 / CPR;
    constexpr int NIW = TB / 1024 / NWV;  // wave loads per wave per tile (K, and again V)
    constexpr int KS = D / 16;            // QK steps (two products each)
    constexpr int EPS = 16 / KS;          // exponentials of a half tile per QK step (2, or 1)
    constexpr int NDT = D / 32;           // 32-column blocks of O
    constexpr int NPV = 4 * NDT;          // PV products per tile (4 key steps x NDT)
    constexpr int PPE = NPV / 16;         // PV products per exponential of a half tile (1, or 2)
    static_assert(NIW >= 1, "tile too small for the waves");
    static_assert(EPS * KS == 16 && PPE * 16 == NPV, "exponentials spread over the products");
    constexpr float kPmax = 256.f;
    // D = 128: the K and V double buffers in one array, so the distance
    // between them is a constant the LDS reads take as their immediate offset
    // (a buffer of its own has an address known only at link time, kept in a
    // register).  At D = 256 the distances pass the 16-bit offset field, and
    // the four buffers stay separate.
    constexpr bool ONE = D == 128;
    __shared__ __attribute__((aligned(1024))) unsigned char sKV[(ONE ? 4 : 1) * TB];
    __shared__ __attribute__((aligned(ONE ? 4 : 1024))) unsigned char sKVb[ONE ? 4 : TB];
    __shared__ __attribute__((aligned(ONE ? 4 : 1024))) unsigned char sKVc[ONE ? 4 : TB];
    __shared__ __attribute__((aligned(ONE ? 4 : 1024))) unsigned char sKVd[ONE ? 4 : TB];
    unsigned char* const sK0 = sKV;
    unsigned char* const sK1 = ONE ? sKV + TB : sKVb;
    unsigned char* const sV0 = ONE ? sKV + 2 * TB : sKVc;
    unsigned char* const sV1 = ONE ? sKV + 3 * TB : sKVd;
    // The boolean mask tile (256 query rows x 64 keys, one byte each).  MASK
    // 3: chunk-major, 16-byte chunk ch of row r at (ch*256 + r)*16; MASK 2:
    // row-major in groups of 4 rows (layout at issue_mask_dwords).  And
    // for MASK 3 the tile classes of the workgroup's rows (two bits per KV
    // tile, the two 128-row summary rows combined), first 64 words.
    constexpr int MT = (MASK == 3) ? 32 * NWV * BN : ((MASK == 2) ? 8 * NWV * 272 : 16);
    __shared__ __attribute__((aligned(1024))) unsigned char sM0[MT];
    __shared__ __attribute__((aligned(1024))) unsigned char sM1[MT];
    __shared__ uint32_t s_cls[(MASK == 3) ? 64 : 1];

    const int tid0 = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid0 >> 6);

    const int64_t units = PERSIST ? a.units : (int64_t)gridDim.x;  // launch slots
    // The arguments as the persistent kernel reads them per unit: scalar
    // loads from the argument segment through an opaque copy of its address,
    // so the compiler keeps none of these values live across the KV loop (the
    // register pressure of that would cost copies inside it).  The kernel's
    // one argument, `a`, starts the segment.
    auto fresh_args = []() __attribute__((always_inline)) -> const __attribute__((address_space(4))) PrefillArgs& {
        auto kp = (const __attribute__((address_space(4))) PrefillArgs*)__builtin_amdgcn_kernarg_segment_ptr();
        asm volatile("" : "+s"(kp));
        return *kp;
    };
    // The unit of work (query tile, head, batch) that launch slot u takes,
    // and the range of keys [kbeg, kv_end) that can be visible to some row of
    // its tile: causal stops at the tile's last row, a window spans from the
    // first row's left edge to the last used row's right edge.
    struct UnitGeom {
        int qt, n1;
        bool valid;
        int64_t b, L;
        int64_t q_used, q_full;    // query rows computed / written
        int64_t q_off, kv_off;     // element offsets of (b) in q/out and k/v
        int64_t lse_row0, lse_step;  // lse index of (n1, row i) = lse_row0 + i * lse_step
        int64_t kbeg, kv_end;
    };
    auto unit_geom = [&](int64_t u, const auto& A) __attribute__((always_inline)) {
        UnitGeom g{};
        g.valid = true;
        g.q_used = A.q_seq;
        g.q_full = A.q_seq;
        // (the persistent kernel of the padded layouts leaves this branch
        // out: compiled in, it cost them 0.5-1 %)
        if ((!PERSIST || PACKED) && A.work) {
            // Packed layout: slot 8k + x (dispatched to XCD x) takes head k % N
            // of work item 8*(k / N) + x, so the heaviest items spread over all
            // XCDs and the heads of one item (which share K/V under GQA) share an L2.
            const int x = (int)(u & 7);
            const int64_t kk = u >> 3;
            const int64_t item = (kk / A.num_heads) * 8 + x;
            g.n1 = (int)(kk % A.num_heads);
            const int32_t wb = item < A.work_items ? A.work[2 * item] : -1;
            if (wb < 0) {
                g.valid = false;
                return g;
            }
            g.b = wb;
            g.qt = A.work[2 * item + 1];
            const SeqGeom sg = seq_geometry(A.cu_q, A.cu_kv, A.used_q, A.lens, g.b, A.batch, A.q_seq, A.kv_seq);
            g.q_used = sg.q_used;
            g.q_full = sg.q_full;
            g.L = sg.kv_len;
            g.q_off = sg.q0 * A.q_stride_s;
            g.kv_off = sg.k0 * A.kv_stride_s;
            g.lse_row0 = sg.q0 * A.num_heads + g.n1;
            g.lse_step = A.num_heads;
        } else {
            // (32-bit unsigned in the persistent kernel, whose launcher keeps
            // the units below 2^31: fewer registers for the divisions)
            using UI = std::conditional_t<PERSIST, uint32_t, int64_t>;
            const UI total = (UI)units, uu = (UI)u, tiles = (UI)A.q_tiles;
            UI bh;
            if (MASK == 1 || MASK == 2 || MASK == 3 || (MASK == 4 && A.win_left >= A.win_right)) {
                // Costs grow with the query tile (causal, a tensor mask that may
                // be causal, or a window reaching further back than forward):
                // every head's tile of one rank is dispatched before the next
                // lighter rank, the heads of a rank spread over the XCDs as below.
                const UI heads = total / tiles;
                g.qt = A.q_tiles - 1 - (int)(uu / heads);
                bh = (UI)xcd_remap((int64_t)(uu % heads), (int64_t)heads);
            } else {
                const UI work = (UI)xcd_remap((int64_t)uu, (int64_t)total);
                g.qt = (int)(work % tiles);
                bh = work / tiles;
            }
            g.n1 = (int)(bh % (UI)A.num_heads);
            g.b = (int64_t)(bh / (UI)A.num_heads);
            g.L = A.kv_seq;
            if (A.lens) {
                const int64_t l = A.lens[g.b];
                g.L = l < 0 ? 0 : (l > A.kv_seq ? A.kv_seq : l);
            }
            if (A.used_q) {  // rows at or past the batch's used positions: written as 0 / +inf
                const int64_t uq = A.used_q[g.b];
                g.q_used = uq < 0 ? 0 : (uq > A.q_seq ? A.q_seq : uq);
            }
            g.q_off = g.b * A.q_stride_b;
            g.kv_off = g.b * A.kv_stride_b;
            g.lse_row0 = (g.b * A.num_heads + g.n1) * A.q_seq;
            g.lse_step = 1;
        }
        const int64_t r0 = (int64_t)g.qt * (32 * NWV);
        g.kv_end = g.L;
        g.kbeg = 0;
        if (MASK == 1 && g.kv_end > r0 + 32 * NWV) g.kv_end = r0 + 32 * NWV;
        if (MASK == 4) {
            const int64_t i_last = (r0 + 32 * NWV < g.q_used ? r0 + 32 * NWV : g.q_used) - 1;
            if (g.kv_end > i_last + A.win_right + 1) g.kv_end = i_last + A.win_right + 1;
            const int64_t key_lo = r0 - A.win_left;
            if (key_lo > 0) g.kbeg = key_lo / BN * BN;
        }
        return g;
    };
    // Q fragments of this lane for the unit (zeros past the used rows; the
    // sign flipped for a negative scale, zeros for a scale that underflows).
    V8 qreg[KS];
    auto load_q = [&](const UnitGeom& gq, int ln, const auto& A) __attribute__((always_inline)) {
        const int64_t row = (int64_t)gq.qt * (32 * NWV) + 32 * wave + (ln & 31);
        const bool ok = row < gq.q_used;
        const uint16_t* qp = A.q + gq.q_off + (int64_t)gq.n1 * A.q_stride_n + row * A.q_stride_s;
        const uint32_t flip = A.negate_q ? 0x80008000u : 0u;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            u32x4 w = u32x4{0u, 0u, 0u, 0u};
            if (ok && !A.zero_q) w = ld128(qp + kk * 16 + 8 * (ln >> 5));
            w ^= flip;
            qreg[kk] = __builtin_bit_cast(V8, w);
        }
    };
    const int64_t row_bytes = a.kv_stride_s * 2;
    const int32_t rb32 = __builtin_amdgcn_readfirstlane((int32_t)row_bytes);
    // A persistent launch (PERSIST) runs one workgroup per CU over the units
    // blockIdx.x, blockIdx.x + gridDim.x, ... (gridDim.x is a multiple of 8,
    // so in these forward rounds every unit keeps the XCD the plain launch
    // would give it); the packed layout's instantiation (PACKED) walks its
    // work list the same way and skips the entries that pad it.  The next
    // unit's Q and first K tile are fetched during the current unit's last
    // slot, which reads neither Q nor a K buffer.
    // Causal costs fall with the rank and the units come heaviest first, so
    // the rounds run forward and backward in turn (a snake): a workgroup's
    // units then sum to about the same cost (ranks 15-r, 8+r, 7-r, r of
    // sixteen in four rounds; with per-batch lengths, nearly so).
    auto slot_unit = [&](int64_t k) __attribute__((always_inline)) -> int64_t {
        const int64_t G = gridDim.x;
        return (PERSIST && MASK == 1 && (k & 1)) ? (k + 1) * G - 1 - (int64_t)blockIdx.x
                                                  : k * G + (int64_t)blockIdx.x;
    };
    int64_t round = 0;  // rounds of gridDim.x units
    int64_t unit = blockIdx.x;
    bool fetched = false;  // Q of `unit` in qreg, its first K tile in sK0
    for (;;) {
        // The persistent kernel produces the lane id afresh for each unit, so
        // neither the thread id nor a value derived from it is kept live
        // across units (which cost copies in the KV loop).
        int lane = tid0 & 63;
        if constexpr (PERSIST) asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
        const int half = lane >> 5;
        const int col = lane & 31;
        const UnitGeom ug = [&]() __attribute__((always_inline)) {
            if constexpr (PERSIST)
                return unit_geom(unit, fresh_args());
            else
                return unit_geom(unit, a);
        }();
        // An entry that pads the packed work list: nothing to compute or write.
        if (!ug.valid) {
            if constexpr (!PERSIST) return;
        }
        const bool live = ug.valid;
        const int qt = ug.qt, n1 = ug.n1;
        const int64_t b = ug.b, L = ug.L, q_used = ug.q_used, q_full = ug.q_full;
        const int64_t q_off = ug.q_off, kv_off = ug.kv_off, lse_row0 = ug.lse_row0, lse_step = ug.lse_step;
        const int n2 = n1 / a.group;

        const int64_t i0 = (int64_t)qt * (32 * NWV);
        const int64_t qrow = i0 + 32 * wave + col;
        const bool qvalid = qrow < q_used;

        if (!fetched && live) {
            if constexpr (PERSIST)
                load_q(ug, lane, fresh_args());
            else
                load_q(ug, lane, a);
        }
        const float c = a.scale_log2;
        int64_t kv_end = ug.kv_end, kbeg = ug.kbeg;
        // MASK 3 with a summary of the mask: the classes of the workgroup's
        // 128-row tiles (two at D = 128), OR-ed (bit 0: some key visible, bit 1:
        // some key masked, for some row), staged for the loop; the first and last
        // tile with a visible key bound the range.  Tiles past the 64 staged
        // words count as partly masked.
        const bool summary = (MASK == 3) && a.mask_cls != nullptr;
        if (MASK == 3 && summary) {
            const int64_t sn = a.mask_stride[1] ? a.num_heads : 1;
            const int64_t slice = (a.mask_stride[0] ? b : 0) * sn + (a.mask_stride[1] ? n1 : 0);
            const int64_t qt128 = (a.q_seq + kMaskRowsPerTile - 1) / kMaskRowsPerTile;
            constexpr int R128 = 32 * NWV / kMaskRowsPerTile;  // summary rows per query tile
            const int64_t r0 = R128 * (int64_t)qt;
            const uint32_t* c0p = a.mask_cls + (slice * qt128 + r0) * a.cls_words;
            const uint32_t* c1p = (R128 == 2 && r0 + 1 < qt128) ? c0p + a.cls_words : nullptr;
            int first = 0x7fffffff, last = -1;
            for (int w = lane; w < a.cls_words; w += 64) {
                const uint32_t x = c0p[w] | (c1p ? c1p[w] : 0u);
                if (w < 64) s_cls[w] = x;  // every wave stages all words (same values), so it reads its own writes
                const uint32_t live = x & 0x55555555u;
                if (live) {
                    first = min(first, 16 * w + (__builtin_ctz(live) >> 1));
                    last = max(last, 16 * w + ((31 - __builtin_clz(live)) >> 1));
                }
            }
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) {
                first = min(first, __shfl_xor(first, off, 64));
                last = max(last, __shfl_xor(last, off, 64));
            }
            first = __builtin_amdgcn_readfirstlane(first);
            last = __builtin_amdgcn_readfirstlane(last);
            if (last < 0) {
                kv_end = 0;  // no visible key for any row
            } else {
                if ((int64_t)first * BN > kbeg) kbeg = (int64_t)first * BN;
                if ((int64_t)(last + 1) * BN < kv_end) kv_end = (int64_t)(last + 1) * BN;
            }
        }
        const int nt = (!live || i0 >= q_used || kv_end <= kbeg) ? 0 : (int)((kv_end - kbeg + BN - 1) / BN);

        f32x16 o[D / 32];
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
        float m_run = kNegInf;  // reference max per query row (scaled base-2 units)
        float l_half = 0.f;     // this half-wave's share of the row sum

        const char* kbase = reinterpret_cast<const char*>(a.k + kv_off + (int64_t)n2 * a.kv_stride_n) + kbeg * row_bytes;
        const char* vbase = reinterpret_cast<const char*>(a.v + kv_off + (int64_t)n2 * a.kv_stride_n) + kbeg * row_bytes;
        int voff[NIW];
#pragma unroll
        for (int w = 0; w < NIW; ++w) {
            const int r = RPI * (wave * NIW + w) + lane / CPR;
            voff[w] = (int)(r * row_bytes) + (((lane % CPR) ^ swz<D>(r)) << 4);
        }
        // Tile loads with their scalars worked out once: the K and V bases of
        // this (b, n2), the bytes per row (a 64-row tile stays below 2^31 bytes,
        // which the host checks), the key count in 32 bits and the LDS address of
        // this wave's share of each buffer; a load then costs a few scalar
        // instructions and the M0 write.
        const uint64_t kb64 = (uint64_t)uni64((int64_t)(uintptr_t)kbase);
        const uint64_t vb64 = (uint64_t)uni64((int64_t)(uintptr_t)vbase);
        const int32_t L32 = __builtin_amdgcn_readfirstlane((int32_t)(kv_end - kbeg));  // keys in the range
        // Visible keys of the wave's first row (wrow0), relative to the range's
        // first key: [c_lo, c_hi] (row wrow0 + col sees [c_lo + col, c_hi + col]),
        // and the bounds [w_lo, w_hi] within which a key is visible to every row of
        // the wave, so a tile inside them needs no per-key mask.  All scalars: the
        // per-lane bounds are rebuilt from the lane id on the masking path only.
        auto clamp_rel = [](int64_t x) __attribute__((always_inline)) {
            return (int32_t)(x < -(int64_t(1) << 30) ? -(int64_t(1) << 30) : (x > (int64_t(1) << 30) ? (int64_t(1) << 30) : x));
        };
        const int64_t wrow0 = i0 + 32 * wave;
        int32_t c_lo = 0, c_hi = L32 - 1;
        if (MASK == 1) c_hi = clamp_rel(wrow0 - kbeg);
        if (MASK == 4) {
            c_lo = clamp_rel(wrow0 - a.win_left - kbeg);
            c_hi = clamp_rel(wrow0 + a.win_right - kbeg);
        }
        c_lo = __builtin_amdgcn_readfirstlane(c_lo);
        c_hi = __builtin_amdgcn_readfirstlane(c_hi);
        const int32_t w_lo = (MASK == 4) ? c_lo + 31 : 0;
        const int32_t w_hi = min(L32 - 1, c_hi);
        const uint32_t wshare = (uint32_t)(wave * NIW * 1024);
        const uint32_t mK0 = lds_address(sK0) + wshare, mK1 = lds_address(sK1) + wshare;
        const uint32_t mV0 = lds_address(sV0) + wshare, mV1 = lds_address(sV1) + wshare;
        // MASK 3 tile loads: wave w fills chunk w%4 (keys 16*(w%4) + [0,16)) of
        // rows 128*(w/4) + [0,128), 64 rows per wave load; the resource stops at
        // the last used row's last key, so nothing past the mask tensor is read.
        const char* mbase = reinterpret_cast<const char*>(a.mask) + b * a.mask_stride[0] +
                            (int64_t)n1 * a.mask_stride[1] + i0 * a.mask_stride[2];
        const int32_t mst2 = __builtin_amdgcn_readfirstlane((int32_t)a.mask_stride[2]);
        int32_t mrec_rows = 0;
        if (MASK == 3) {
            int64_t rv = q_used - i0;
            rv = rv > 32 * NWV ? 32 * NWV : rv;
            mrec_rows = __builtin_amdgcn_readfirstlane((int32_t)((rv - 1) * a.mask_stride[2]));
        }
        const uint32_t mM0 = lds_address(sM0) + (uint32_t)((wave & 3) * (32 * NWV) + 128 * (wave >> 2)) * 16u;
        const uint32_t mM1 = lds_address(sM1) + (uint32_t)((wave & 3) * (32 * NWV) + 128 * (wave >> 2)) * 16u;
        // Class of tile jl, asked for in increasing order: the staged word of the
        // current 16 tiles is kept in a scalar and read from LDS once per word
        // (an LDS read here would make the slot wait for its in-flight K reads).
        uint32_t cword = 0u;
        int cw_idx = -1;
        auto tile_cls = [&](int jl) __attribute__((always_inline)) -> uint32_t {
            const int64_t jt = kbeg / BN + jl;
            if (!summary || jt >= 64 * 16) return 3u;
            const int wi = (int)(jt >> 4);
            if (wi != cw_idx) {
                cword = __builtin_amdgcn_readfirstlane(s_cls[wi]);
                cw_idx = wi;
            }
            return (cword >> (2 * (jt & 15))) & 3u;
        };
        uint32_t cls_cur = 3u, cls_nxt = 3u;  // classes of tiles j and j+1 in slot j
        // MASK 2 tile loads (rows of 4-aligned key runs): four keys per lane, one
        // group of 4 rows per wave load (lane l: row 4G + l/16, keys 4(l%16) +
        // [0, 4)), wave w loading groups 8w .. 8w+7 (its own rows); group G sits at
        // G*272 in LDS, rows 64 bytes apart (the 16-byte step between groups
        // spreads a wave's reads over the banks).  Each group's resource stops at
        // its last used row's last key; groups with no used row are not loaded.
        constexpr int MGP = 272;
        const uint32_t mE0 = lds_address(sM0) + (uint32_t)(8 * wave * MGP);
        const uint32_t mE1 = lds_address(sM1) + (uint32_t)(8 * wave * MGP);
        auto issue_mask_dwords = [&](int jl, uint32_t m0) __attribute__((always_inline)) {
            const int64_t j0 = kbeg + (int64_t)jl * BN;
            int64_t keys = a.kv_seq - j0;
            keys = keys > BN ? BN : keys;
            const int ln = (int)__lane_id();
            const int voff = (ln >> 4) * mst2 + (ln & 15) * 4;
            const uint64_t gb = (uint64_t)(uintptr_t)(mbase + j0) + (uint64_t)(int64_t)(32 * wave) * (uint64_t)(int64_t)mst2;
            const int32_t rows = __builtin_amdgcn_readfirstlane((int32_t)(q_used - i0 - 32 * wave));
#pragma unroll
            for (int G = 0; G < 8; ++G) {
                const int32_t rv = min(rows - 4 * G, 4);
                if (rv <= 0) break;
                const uint64_t t = gb + (uint64_t)(int64_t)(4 * G) * (uint64_t)(int64_t)mst2;
                dma_rsrc r;
                r[0] = (uint32_t)t;
                r[1] = (uint32_t)(t >> 32) & 0xffffu;
                r[2] = (uint32_t)((rv - 1) * mst2 + (int32_t)keys);
                r[3] = 0x00020000u;
                lds_dma4_m0(r, m0 + (uint32_t)(G * MGP), voff);
            }
        };
        auto issue_mask = [&](int jl, uint32_t cls, uint32_t m0) __attribute__((always_inline)) {
            if (!(cls & 2u)) return;  // no key masked (or none visible): nothing to stage
            const int64_t j0 = kbeg + (int64_t)jl * BN;
            int64_t keys = a.kv_seq - j0;
            keys = keys > BN ? BN : keys;
            const dma_rsrc rm = make_dma_rsrc(mbase + j0, mrec_rows + (int)keys);
            const int ln = (int)__lane_id();
#pragma unroll
            for (int w = 0; w < 2; ++w)
                lds_dma16_m0(rm, m0 + (uint32_t)(w * 1024),
                             (128 * (wave >> 2) + 64 * w + ln) * mst2 + (wave & 3) * 16);
        };
        // Bytes of a full tile, and of the last one (cut at the length).
        const uint32_t full_bytes = (uint32_t)(BN * rb32);
        const uint32_t last_bytes = (uint32_t)((L32 - (nt - 1) * BN) * rb32);
        auto issue_at = [&](uint64_t t, uint32_t bytes, uint32_t m0) __attribute__((always_inline)) {
            dma_rsrc r;
            r[0] = (uint32_t)t;
            r[1] = (uint32_t)(t >> 32) & 0xffffu;
            r[2] = bytes;
            r[3] = 0x00020000u;
#pragma unroll
            for (int w = 0; w < NIW; ++w) lds_dma16_m0(r, m0 + (uint32_t)(w * 1024), voff[w]);
        };
        auto issue = [&](uint64_t base, int jt, uint32_t m0) __attribute__((always_inline)) {
            issue_at(base + (uint64_t)(uint32_t)jt * (uint64_t)full_bytes, jt + 1 < nt ? full_bytes : last_bytes, m0);
        };
        // Persistent launch, before the last slot: Q of the next unit into qreg
        // and its first K tile into sK0.
        auto fetch_next = [&]() __attribute__((always_inline)) {
            const int64_t nu = slot_unit(round + 1);
            if (nu >= units) return;
            const auto& A = fresh_args();
            const UnitGeom gn = unit_geom(nu, A);
            if (!gn.valid) return;
            int ln;  // the lane id produced here, not kept live from the unit's start
            asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
            load_q(gn, ln, A);
            const int64_t nkeys = gn.kv_end - gn.kbeg;
            if ((int64_t)gn.qt * (32 * NWV) < gn.q_used && nkeys > 0) {
                const char* kb = reinterpret_cast<const char*>(A.k + gn.kv_off + (int64_t)(gn.n1 / A.group) * A.kv_stride_n) +
                                 gn.kbeg * row_bytes;
                const int32_t rows = __builtin_amdgcn_readfirstlane((int32_t)(nkeys < BN ? nkeys : BN));
                issue_at((uint64_t)uni64((int64_t)(uintptr_t)kb), (uint32_t)(rows * rb32), mK0);
            }
            fetched = true;
        };

        // LDS read addressing, as in the other prefill kernels.
        const int krow0 = col, krow1 = 32 + col;
        const int ks0 = swz<D>(krow0), ks1 = swz<D>(krow1);
        const int trG = lane >> 4;
        const int trL = lane & 15;
        const int vrow_lo = 4 * (trG >> 1) + (trL >> 2);
        const int vrow_hi = vrow_lo + 8;
        const int vs_lo = swz<D>(vrow_lo), vs_hi = swz<D>(vrow_hi);
        const int vx = 2 * (trG & 1) + ((trL & 3) >> 1);
        const int vbyte = (trL & 1) * 8;
        auto kread = [&](const unsigned char* Kb, int kk, V8* dst) __attribute__((always_inline)) {
            dst[0] = __builtin_bit_cast(V8, *reinterpret_cast<const u32x4*>(Kb + krow0 * RB + (((2 * kk + half) ^ ks0) << 4)));
            dst[1] = __builtin_bit_cast(V8, *reinterpret_cast<const u32x4*>(Kb + krow1 * RB + (((2 * kk + half) ^ ks1) << 4)));
        };
        // V^T operand of product (ks, dt): keys 16*ks + .., head-dim columns 32*dt + ..
        auto vread = [&](const unsigned char* Vb, int i) __attribute__((always_inline)) -> V8 {
            const int ks = i / NDT, dt = i % NDT;
            const int lc = 4 * dt + vx;
            const unsigned char* vb = Vb + ks * 16 * RB;
            const s16x4 lo = lds_read_tr(vb + vrow_lo * RB + ((lc ^ vs_lo) << 4) + vbyte);
            const s16x4 hi = lds_read_tr(vb + vrow_hi * RB + ((lc ^ vs_hi) << 4) + vbyte);
            return __builtin_bit_cast(V8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        const f32x16 zero16 = {};

        // Stage A of a slot: S(j) into Sn (when QK), exponentials of the second
        // half of tile j-1 (So[1]) into Pd[2..3] and their sum ps1 (when SM).
        auto stage_a = [&](auto qk_t, auto sm_t, const unsigned char* Kb, f32x16* Sn, const f32x16* So, u32x4* Pd,
                           float& ps1) __attribute__((always_inline)) {
            constexpr bool QK = decltype(qk_t)::value;
            constexpr bool SM = decltype(sm_t)::value;
            const float nmx = (m_run == kNegInf) ? 0.f : -m_run;
            constexpr int PF = 2;  // K fragments read two steps ahead
            V8 kring[PF + 1][2];
            if constexpr (QK) {
#pragma unroll
                for (int p = 0; p < PF; ++p) kread(Kb, p, kring[p]);
            }
            float acc = 0.f, pprev = 0.f;
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                if constexpr (QK) {
                    if (kk + PF < KS) kread(Kb, kk + PF, kring[(kk + PF) % (PF + 1)]);
                }
                // each step in this order: fragment reads, vector work, products
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (SM && EPS == 2) {
                    const int r = 2 * kk;
                    const float p0 = fast_exp2(__builtin_fmaf(So[1][r], c, nmx));
                    const float p1 = fast_exp2(__builtin_fmaf(So[1][r + 1], c, nmx));
                    acc += p0;
                    acc += p1;
                    uint32_t w = cvt_pair<ST>(p0, p1);
                    // keep the sum and the conversion in this step (the compiler
                    // would otherwise sink them past the products)
                    asm volatile("" : "+v"(acc), "+v"(w));
                    Pd[2 + (r >> 3)][(r & 7) >> 1] = w;
                } else if constexpr (SM) {  // one exponential per step, converted in pairs
                    const int r = kk;
                    const float p = fast_exp2(__builtin_fmaf(So[1][r], c, nmx));
                    acc += p;
                    if (r & 1) {
                        uint32_t w = cvt_pair<ST>(pprev, p);
                        asm volatile("" : "+v"(acc), "+v"(w));
                        Pd[2 + (r >> 3)][(r & 7) >> 1] = w;
                    } else {
                        pprev = p;
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (QK) {
                    const V8* kf = kring[kk % (PF + 1)];
                    // Two waves share a SIMD at D = 128: the one issuing products takes
                    // priority, which keeps the matrix core fed (at D = 256, one wave per
                    // SIMD, the priority change only costs).
                    if constexpr (NWV == 8) __builtin_amdgcn_s_setprio(1);
                    Sn[0] = M::mm(kf[0], qreg[kk], kk == 0 ? zero16 : Sn[0]);
                    Sn[1] = M::mm(kf[1], qreg[kk], kk == 0 ? zero16 : Sn[1]);
                    if constexpr (NWV == 8) __builtin_amdgcn_s_setprio(0);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (SM) ps1 = acc;
        };
        // Stage B: O += V(j-1)^T P(j-1) (when PV, Po = P(j-1)), exponentials of
        // the first half of tile j (Sn[0]) into Pn[0..1] and their sum ps0 (when SM).
        auto stage_b = [&](auto pv_t, auto sm_t, const unsigned char* Vb, const u32x4* Po, const f32x16* Sn, u32x4* Pn,
                           float& ps0) __attribute__((always_inline)) {
            constexpr bool PV = decltype(pv_t)::value;
            constexpr bool SM = decltype(sm_t)::value;
            const float nmx = (m_run == kNegInf) ? 0.f : -m_run;
            constexpr int VPF = 3;  // V operands read three products ahead
            V8 vring[VPF + 1];
            if constexpr (PV) {
#pragma unroll
                for (int p = 0; p < VPF; ++p) vring[p] = vread(Vb, p);
            }
            float acc = 0.f, pprev = 0.f;
#pragma unroll
            for (int i = 0; i < NPV; ++i) {
                if constexpr (PV) {
                    if (i + VPF < NPV) vring[(i + VPF) % (VPF + 1)] = vread(Vb, i + VPF);
                }
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (SM) {
                    if (i % PPE == 0) {
                        const int e = i / PPE;
                        const float p = fast_exp2(__builtin_fmaf(Sn[0][e], c, nmx));
                        acc += p;
                        if (e & 1) {
                            uint32_t w = cvt_pair<ST>(pprev, p);
                            asm volatile("" : "+v"(acc), "+v"(w));
                            Pn[e >> 3][(e & 7) >> 1] = w;
                        } else {
                            pprev = p;
                        }
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (PV) {
                    if constexpr (NWV == 8) __builtin_amdgcn_s_setprio(1);
                    o[i % NDT] = M::mm(vring[i % (VPF + 1)], __builtin_bit_cast(V8, Po[i / NDT]), o[i % NDT]);
                    if constexpr (NWV == 8) __builtin_amdgcn_s_setprio(0);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (SM) ps0 = acc;
        };
        // Rare paths.  After stage B, the first half of tile j exceeded its bound
        // (or the row has seen no key yet): the reference moves to the maximum of
        // the whole tile, so its second half cannot exceed it later; O (which
        // holds tile j-1 by then) and the row sum are rescaled, and the first
        // half's exponentials are taken again.
        auto rescale_b = [&](const f32x16* St, u32x4* Pt, float& ps0) __attribute__((always_inline)) {
            float tmax = kNegInf;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, St[tt][r]);
            tmax = fmaxf(tmax, xor32(tmax)) * c;
            const float mnew = fmaxf(m_run, tmax);
            const float alpha = fast_exp2(m_run - ((mnew == kNegInf) ? 0.f : mnew));
            scale_acc<D>(o, alpha);
            l_half *= alpha;
            m_run = mnew;
            const float nmx = (m_run == kNegInf) ? 0.f : -m_run;
            float s0 = 0.f;
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float p0 = fast_exp2(__builtin_fmaf(St[0][r], c, nmx));
                const float p1 = fast_exp2(__builtin_fmaf(St[0][r + 1], c, nmx));
                s0 += p0;
                s0 += p1;
                Pt[r >> 3][(r & 7) >> 1] = cvt_pair<ST>(p0, p1);
            }
            ps0 = s0;
        };
        // After stage A, the second half of tile j-1 exceeded its bound (its
        // first half passed, so its scores lie below the reference + 8): the
        // reference moves to the second half's maximum, O (tiles before j-1) and
        // the row sum are rescaled, the second half's exponentials are taken
        // again and the first half's 16-bit values and sum are scaled by the same
        // factor (at most one more rounding of those values, on this rare path).
        auto rescale_a = [&](const f32x16* St, u32x4* Pt, float& ps0, float& ps1) __attribute__((always_inline)) {
            float tmax = kNegInf;
#pragma unroll
            for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, St[1][r]);
            tmax = fmaxf(tmax, xor32(tmax)) * c;
            const float mnew = fmaxf(m_run, tmax);
            // (a row that has seen no key yet -- a window's left edge, rows a
            // wave shares -- keeps the reference -inf and exponentials against 0)
            const float alpha = fast_exp2(m_run - ((mnew == kNegInf) ? 0.f : mnew));
            scale_acc<D>(o, alpha);
            l_half *= alpha;
            m_run = mnew;
            const float nmx = (m_run == kNegInf) ? 0.f : -m_run;
            float s1 = 0.f;
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float p0 = fast_exp2(__builtin_fmaf(St[1][r], c, nmx));
                const float p1 = fast_exp2(__builtin_fmaf(St[1][r + 1], c, nmx));
                s1 += p0;
                s1 += p1;
                Pt[2 + (r >> 3)][(r & 7) >> 1] = cvt_pair<ST>(p0, p1);
            }
            ps1 = s1;
#pragma unroll
            for (int wd = 0; wd < 8; ++wd) {
                const uint32_t x = Pt[wd >> 2][wd & 3];
                Pt[wd >> 2][wd & 3] = cvt_pair<ST>(lo_f32<ST>(x) * alpha, hi_f32<ST>(x) * alpha);
            }
            ps0 *= alpha;
        };

        f32x16 SA[2], SB[2];
        u32x4 PA[4], PB[4];
        float ps0 = 0.f, ps1 = 0.f;
        // Slot j (PAR = j & 1): K(j) in sK[PAR], V(j-1) in sV[PAR ^ 1]; tiles
        // j+1 (K) and j (V) are fetched into the other buffers.  S(j) goes to
        // SA for even j, SB for odd j; P(j) likewise to PA / PB.
        auto slot = [&](auto par_t, auto first_t, auto last_t, int j) __attribute__((always_inline)) {
            constexpr int PAR = decltype(par_t)::value;
            constexpr bool FIRST = decltype(first_t)::value;  // j == 0: no tile j-1
            constexpr bool LAST = decltype(last_t)::value;    // j == nt: no tile j
            const unsigned char* Kc = PAR ? sK1 : sK0;
            const unsigned char* Vp = PAR ? sV0 : sV1;
            const uint32_t mKn = PAR ? mK0 : mK1;
            const uint32_t mVn = PAR ? mV1 : mV0;
            const unsigned char* Mc = PAR ? sM1 : sM0;  // MASK 2, 3: mask tile j
            const uint32_t mMn = PAR ? mM0 : mM1;       // ... and where tile j+1's goes
            const uint32_t mEn = PAR ? mE0 : mE1;
            f32x16* Sn = PAR ? SB : SA;
            f32x16* So = PAR ? SA : SB;
            u32x4* Pn = PAR ? PB : PA;
            u32x4* Po = PAR ? PA : PB;
            // K(j+1) now and V(j) after stage A, into the buffers the previous
            // slot released (issued together, the 8 waves' loads queue for the
            // address unit at the slot's start)
            if (j + 1 < nt) {
                issue(kb64, j + 1, mKn);
                if constexpr (MASK == 3) {
                    cls_nxt = tile_cls(j + 1);
                    issue_mask(j + 1, cls_nxt, mMn);
                }
                if constexpr (MASK == 2) issue_mask_dwords(j + 1, mEn);
            }
            stage_a(std::integral_constant<bool, !LAST>{}, std::integral_constant<bool, !FIRST>{}, Kc, Sn, So, Po, ps1);
            if (j < nt) issue(vb64, j, mVn);
            if constexpr (!FIRST) {
                // second half of tile j-1 above its bound: rare rescale, then the
                // row sum takes the whole tile
                if (__any(ps1 > kPmax)) rescale_a(So, Po, ps0, ps1);
                l_half += ps0 + ps1;
            }
            if constexpr (!LAST) {
                // Keys past the range (the last tile), and for the masks the tiles
                // that cross the diagonal or a band edge of one of the wave's rows:
                // the excluded keys' scores become -inf.
                const int32_t j0 = j * BN;
                uint32_t tcls = 3u;
                if constexpr (MASK == 3) tcls = cls_cur;
                // One block changes the scores (a single changed path lets the
                // compiler keep them in the registers the products wrote; with a
                // second one, every tile paid 32 copies where the paths join).
                if (MASK == 2 || (MASK == 3 && (tcls != 1u || j0 + BN - 1 > w_hi))) {
                    // the staged mask tile (MASK 3: when the tile's class says a
                    // key is masked): word (tt, g) of this lane holds keys
                    // 32*tt + 8*g + 4*half + [0, 4) of its row; keys past the
                    // range are excluded too.  A tile with no key visible to any
                    // row of the workgroup (class bit 0 clear) is excluded whole,
                    // whether or not its mask was staged.
                    const int ln = (int)__lane_id();
                    const int row = 32 * wave + (ln & 31), h4 = (ln >> 5) * 4;
                    const int32_t hi = (MASK == 3 && !(tcls & 1u)) ? -0x7fffffff : L32 - 1 - j0 - h4;
                    const bool staged = MASK == 2 || (tcls & 2u);
#pragma unroll
                    for (int tt = 0; tt < 2; ++tt) {
                        uint32_t mw[4] = {0u, 0u, 0u, 0u};
                        if (staged) {
#pragma unroll
                            for (int g = 0; g < 4; ++g) {
                                if constexpr (MASK == 3)
                                    mw[g] = *reinterpret_cast<const uint32_t*>(
                                        Mc + ((2 * tt + (g >> 1)) * (32 * NWV) + row) * 16 + 8 * (g & 1) + h4);
                                else
                                    mw[g] = *reinterpret_cast<const uint32_t*>(Mc + (row >> 2) * 272 + (row & 3) * 64 +
                                                                               32 * tt + 8 * g + h4);
                            }
                        }
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int32_t e = tt * 32 + 8 * (r >> 2) + (r & 3);
                            const bool ok = e <= hi && ((mw[r >> 2] >> (8 * (r & 3))) & 0xffu) == 0u;
                            Sn[tt][r] = ok ? Sn[tt][r] : kNegInf;
                        }
                    }
                } else if (MASK != 2 && MASK != 3 && (j0 < w_lo || j0 + BN - 1 > w_hi)) {
                    // element (tt, r) is key j0 + e + 4*half, e = 32tt + 8(r/4) + r%4
                    const int ln = (int)__lane_id();
                    const int cl = ln & 31, h4 = (ln >> 5) * 4;
                    int32_t hi = L32 - 1 - j0;
                    if (MASK != 0) hi = min(hi, c_hi - j0 + cl);
                    hi -= h4;
                    const int32_t lo = c_lo - j0 + cl - h4;
#pragma unroll
                    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int32_t e = tt * 32 + 8 * (r >> 2) + (r & 3);
                            const bool ok = e <= hi && (MASK != 4 || e >= lo);
                            Sn[tt][r] = ok ? Sn[tt][r] : kNegInf;
                        }
                }
            }
            stage_b(std::integral_constant<bool, !FIRST>{}, std::integral_constant<bool, !LAST>{}, Vp, Po, Sn, Pn, ps0);
            if constexpr (!LAST) {
                // first half of tile j above its bound, or a row that has seen no
                // key yet: rare rescale against the whole tile's maximum
                if (__any(ps0 > kPmax || (m_run == kNegInf && qvalid))) rescale_b(Sn, Pn, ps0);
            }
            if constexpr (MASK == 3) cls_cur = cls_nxt;
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's loads of slot j+1 landed
            __syncthreads();                                   // ... and everyone else's
        };
        using T0 = std::integral_constant<int, 0>;
        using T1 = std::integral_constant<int, 1>;
        using BT = std::true_type;
        using BF = std::false_type;

        const bool have_k0 = fetched;
        fetched = false;
        if (nt > 0) {
            if (!have_k0) {
                issue(kb64, 0, mK0);
                if constexpr (MASK == 3) {
                    cls_cur = tile_cls(0);
                    issue_mask(0, cls_cur, mM0);
                }
                if constexpr (MASK == 2) issue_mask_dwords(0, mE0);
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                __syncthreads();
            }
            slot(T0{}, BT{}, BF{}, 0);
            int j = 1;
            for (; j + 1 < nt; j += 2) {
                slot(T1{}, BF{}, BF{}, j);
                slot(T0{}, BF{}, BF{}, j + 1);
            }
            if (j < nt) {
                slot(T1{}, BF{}, BF{}, j);
                ++j;
            }
            if constexpr (PERSIST) fetch_next();
            if (nt & 1)
                slot(T1{}, BF{}, BT{}, nt);
            else
                slot(T0{}, BF{}, BT{}, nt);
        }

        const float l_run = l_half + xor32(l_half);
        if (live && qrow < q_full) {
            const bool empty = !qvalid || (m_run == kNegInf);
            const float inv = empty ? 0.f : 1.f / l_run;
            uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + q_off + (int64_t)n1 * a.q_stride_n + qrow * a.q_stride_s;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
                for (int a4 = 0; a4 < 4; ++a4) {
                    const int d0 = dt * 32 + 8 * a4 + 4 * half;
                    float x[4];
#pragma unroll
                    for (int cc = 0; cc < 4; ++cc) x[cc] = empty ? 0.f : o[dt][4 * a4 + cc] * inv;
                    u32x2 w;
                    w[0] = pack2<ST>(x[0], x[1]);
                    w[1] = pack2<ST>(x[2], x[3]);
                    *reinterpret_cast<u32x2*>(op + d0) = w;
                }
            }
            if (half == 0 && a.lse) a.lse[lse_row0 + qrow * lse_step] = empty ? kPosInf : (m_run + log2f(l_run)) * kLn2;
        }
        if constexpr (!PERSIST) return;
        unit = slot_unit(++round);
        if (unit >= units) return;
    }  // units
}

template <typename ST, int D>
static hipError_t dispatch_prefill(const PrefillArgs& a, int mask_mode, int64_t blocks, hipStream_t s) {
    const dim3 grid((unsigned)blocks), block(256);
    switch (mask_mode) {
        case 0: hipLaunchKernelGGL((prefill_kernel<ST, D, 0>), grid, block, 0, s, a); break;
        case 1: hipLaunchKernelGGL((prefill_kernel<ST, D, 1>), grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL((prefill_kernel<ST, D, 2>), grid, block, 0, s, a); break;
        case 3: hipLaunchKernelGGL((prefill_kernel<ST, D, 3>), grid, block, 0, s, a); break;
        case 4: hipLaunchKernelGGL((prefill_kernel<ST, D, 4>), grid, block, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

int64_t prefill_persistent_grid(int head_dim, int mask_mode, int64_t units, int cus) {
    if (head_dim != 128) return 0;
    if (!(mask_mode == 0 || mask_mode == 1 || mask_mode == 4)) return 0;
    const int64_t grid = (int64_t)(cus / 8) * 8;
    return (grid >= 8 && units > grid) ? grid : 0;
}

template <typename ST, int D, bool P, bool PK = false>
static void launch_il_mask(const PrefillArgs& a, int mask_mode, dim3 grid, dim3 block, hipStream_t s) {
    switch (mask_mode) {
        case 0: hipLaunchKernelGGL((prefill_il_kernel<ST, D, 0, P, PK>), grid, block, 0, s, a); break;
        case 1: hipLaunchKernelGGL((prefill_il_kernel<ST, D, 1, P, PK>), grid, block, 0, s, a); break;
        case 4: hipLaunchKernelGGL((prefill_il_kernel<ST, D, 4, P, PK>), grid, block, 0, s, a); break;
        default:
            if constexpr (!P) {
                switch (mask_mode) {
                    case 2: hipLaunchKernelGGL((prefill_il_kernel<ST, D, 2, false>), grid, block, 0, s, a); break;
                    case 3: hipLaunchKernelGGL((prefill_il_kernel<ST, D, 3, false>), grid, block, 0, s, a); break;
                }
            }
    }
}

template <typename ST, int D>
static hipError_t launch_il(const PrefillArgs& a0, int mask_mode, int64_t batch, hipStream_t s) {
    constexpr int R = 32 * il_waves<D>();  // query rows per workgroup
    if (mask_mode < 0 || mask_mode > 4) return hipErrorInvalidValue;
    PrefillArgs a = a0;
    a.q_tiles = (int32_t)((a.q_seq + R - 1) / R);
    const int64_t units = a.work ? (int64_t)(a.work_items + 7) / 8 * 8 * a.num_heads
                                 : (int64_t)a.q_tiles * batch * a.num_heads;
    if (units <= 0) return hipSuccess;
    if (units > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    a.units = units;
    const int64_t pgrid = prefill_persistent_grid(D, mask_mode, units, a.cus);
    const dim3 block(2 * R);
    if constexpr (D == 128) {
        if (pgrid > 0) {
            if (a.work)
                launch_il_mask<ST, D, true, true>(a, mask_mode, dim3((unsigned)pgrid), block, s);
            else
                launch_il_mask<ST, D, true>(a, mask_mode, dim3((unsigned)pgrid), block, s);
            return hipGetLastError();
        }
    }
    launch_il_mask<ST, D, false>(a, mask_mode, dim3((unsigned)units), block, s);
    return hipGetLastError();
}

// The interleaved kernel takes head dims 128 and 256 with every mask kind
// but a boolean tensor read element by element.
bool prefill_interleaved(int head_dim, int mask_mode, bool mask_dwords) {
    return (head_dim == 128 || head_dim == 256) && !(mask_mode == 2 && !mask_dwords);
}

int prefill_rows_per_tile(int head_dim, int mask_mode, bool mask_dwords) {
    if (!prefill_interleaved(head_dim, mask_mode, mask_dwords)) return 128;
    return head_dim == 256 ? 32 * il_waves<256>() : 32 * il_waves<128>();
}

hipError_t launch_prefill(const PrefillArgs& a, int dtype, int head_dim, int mask_mode, int64_t batch,
                          hipStream_t stream) {
    if (prefill_interleaved(head_dim, mask_mode, a.mask_dwords != 0)) {
        if (a.q_seq <= 0 || batch <= 0) return hipSuccess;
        if (head_dim == 256)
            return dtype == 1 ? launch_il<BF16, 256>(a, mask_mode, batch, stream)
                              : launch_il<F16, 256>(a, mask_mode, batch, stream);
        return dtype == 1 ? launch_il<BF16, 128>(a, mask_mode, batch, stream)
                          : launch_il<F16, 128>(a, mask_mode, batch, stream);
    }
    const int64_t blocks = a.work ? (int64_t)(a.work_items + 7) / 8 * 8 * a.num_heads
                                  : (int64_t)a.q_tiles * batch * a.num_heads;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (dtype == 1) {
        if (head_dim == 128) return dispatch_prefill<BF16, 128>(a, mask_mode, blocks, stream);
        if (head_dim == 64) return dispatch_prefill<BF16, 64>(a, mask_mode, blocks, stream);
        if (head_dim == 256) return dispatch_prefill<BF16, 256>(a, mask_mode, blocks, stream);
    } else {
        if (head_dim == 128) return dispatch_prefill<F16, 128>(a, mask_mode, blocks, stream);
        if (head_dim == 64) return dispatch_prefill<F16, 64>(a, mask_mode, blocks, stream);
        if (head_dim == 256) return dispatch_prefill<F16, 256>(a, mask_mode, blocks, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace fa
