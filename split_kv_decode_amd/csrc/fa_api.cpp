// fa_api.cpp -- the C ABI declared in include/fa.h: parameter validation
// (complete before anything is enqueued), the split-KV planner and dispatch to
// the gfx950 kernels.  Host-only code; it never allocates device memory and
// never synchronises.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "fa.h"
#include "fa_kernels.h"

// Scratch memory of fa_fwd_noalloc (16 MiB per GPU; see scratch_address).
constexpr size_t kNoallocScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {

thread_local std::string g_last_error;

fa_status fail(fa_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

fa_status ok() { return FA_OK; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Largest products stay far below 2^62 for any accepted shape.
constexpr int64_t kMaxDim = int64_t(1) << 31;
constexpr int64_t kMaxElems = int64_t(1) << 40;
constexpr int64_t kMaxSplits = 1 << 20;

struct Shape {
    int64_t B, QN, KVN, QS, KVS, D, g;
};

bool fast_decode(const fa_params* p);
bool vector_masked_decode(const fa_params* p, const Shape& s);
bool general_split_ok(const fa_params* p, const Shape& s);
int row_groups(const Shape& s);
int prefill_mask_kind(const fa_params* p, const Shape& s);
bool mask_in_dwords(const fa_params* p, const Shape& s);

fa_status check_params(const fa_params* p, Shape* s) {
    if (!p) return fail(FA_ERR_NULLPTR, "params is NULL");
    if (p->batch < 1 || p->batch >= kMaxDim) return fail(FA_ERR_PARAM_INVALID, "batch must be in [1, 2^31), got %lld", (long long)p->batch);
    if (p->num_heads < 1 || p->num_heads >= kMaxDim)
        return fail(FA_ERR_PARAM_INVALID, "num_heads must be in [1, 2^31), got %lld", (long long)p->num_heads);
    if (p->num_kv_heads < 0 || p->num_kv_heads >= kMaxDim)
        return fail(FA_ERR_PARAM_INVALID, "num_kv_heads must be >= 0, got %lld", (long long)p->num_kv_heads);
    const int64_t kvn = p->num_kv_heads == 0 ? p->num_heads : p->num_kv_heads;
    if (p->num_heads % kvn != 0)
        return fail(FA_ERR_PARAM_INVALID, "num_heads (%lld) must be a multiple of num_kv_heads (%lld)",
                    (long long)p->num_heads, (long long)kvn);
    if (p->q_seq < 1 || p->q_seq >= kMaxDim) return fail(FA_ERR_PARAM_INVALID, "q_seq must be in [1, 2^31), got %lld", (long long)p->q_seq);
    if (p->kv_seq < 1 || p->kv_seq >= kMaxDim) return fail(FA_ERR_PARAM_INVALID, "kv_seq must be in [1, 2^31), got %lld", (long long)p->kv_seq);
    if (p->head_dim != 64 && p->head_dim != 128 && p->head_dim != 256) {
        if (p->head_dim > 0 && p->head_dim <= 512 && p->head_dim % 16 == 0)
            return fail(FA_ERR_UNSUPPORTED, "head_dim %lld is not built (64, 128 and 256 are)", (long long)p->head_dim);
        return fail(FA_ERR_PARAM_INVALID, "head_dim must be a positive multiple of 16 up to 512, got %lld",
                    (long long)p->head_dim);
    }
    if (p->layout != FA_BNSD && p->layout != FA_BSND && p->layout != FA_TND)
        return fail(FA_ERR_PARAM_INVALID, "unknown layout %d", (int)p->layout);
    if (p->layout == FA_TND) {
        if (!p->cu_seqlens_q || !p->cu_seqlens_kv)
            return fail(FA_ERR_NULLPTR, "the TND layout needs cu_seqlens_q and cu_seqlens_kv");
        if (p->batch > fa::kVarlenMaxBatch)
            return fail(FA_ERR_PARAM_INVALID, "the TND layout takes at most %d sequences, got %lld",
                        fa::kVarlenMaxBatch, (long long)p->batch);
        if (p->kv_layout != FA_KV_CONTIGUOUS)
            return fail(FA_ERR_UNSUPPORTED, "a paged KV cache with the TND layout is not built");
        if (p->mask_mode == FA_MASK_BOOL)
            return fail(FA_ERR_UNSUPPORTED, "a boolean mask tensor with the TND layout is not built");
    } else if (p->cu_seqlens_q || p->cu_seqlens_kv) {
        return fail(FA_ERR_PARAM_INVALID, "cu_seqlens_q / cu_seqlens_kv are for the TND layout only");
    }
    if (p->dtype != FA_F16 && p->dtype != FA_BF16) return fail(FA_ERR_PARAM_INVALID, "unknown dtype %d", (int)p->dtype);
    if (!std::isfinite(p->scale)) return fail(FA_ERR_PARAM_INVALID, "scale must be finite");
    // The kernels scale scores by scale * log2(e) in fp32.
    if (!std::isfinite((float)(std::fabs(p->scale) * 1.4426950408889634)))
        return fail(FA_ERR_PARAM_INVALID, "|scale| * log2(e) must be finite in fp32, got scale %g", p->scale);
    if (p->mask_mode != FA_MASK_NONE && p->mask_mode != FA_MASK_CAUSAL && p->mask_mode != FA_MASK_BOOL &&
        p->mask_mode != FA_MASK_WINDOW)
        return fail(FA_ERR_PARAM_INVALID, "unknown mask_mode %d", (int)p->mask_mode);
    if (p->mask_mode == FA_MASK_WINDOW && (p->win_left < -1 || p->win_right < -1))
        return fail(FA_ERR_PARAM_INVALID, "win_left and win_right must be >= -1 (-1 = unbounded), got %lld, %lld",
                    (long long)p->win_left, (long long)p->win_right);
    // FlashAttn developer guide 1.5: without the window mode the two bounds are -1.
    if (p->mask_mode != FA_MASK_WINDOW && (p->win_left != -1 || p->win_right != -1))
        return fail(FA_ERR_PARAM_INVALID, "win_left and win_right must be -1 outside the window mode, got %lld, %lld",
                    (long long)p->win_left, (long long)p->win_right);
    if (p->mask_mode == FA_MASK_BOOL && !p->mask) return fail(FA_ERR_NULLPTR, "mask_mode BOOL needs a mask tensor");
    if (p->mask_mode != FA_MASK_BOOL && p->mask)
        return fail(FA_ERR_PARAM_INVALID, "a mask tensor was passed but mask_mode is not BOOL");
    if (p->mask_mode == FA_MASK_BOOL)
        for (int i = 0; i < 4; ++i)
            if (p->mask_stride[i] < 0) return fail(FA_ERR_PARAM_INVALID, "mask strides must be >= 0");
    if (p->kv_layout != FA_KV_CONTIGUOUS && p->kv_layout != FA_KV_PAGED_BBND && p->kv_layout != FA_KV_PAGED_BNBD)
        return fail(FA_ERR_PARAM_INVALID, "unknown kv_layout %d", (int)p->kv_layout);
    if (p->kv_layout == FA_KV_CONTIGUOUS) {
        if (p->block_table) return fail(FA_ERR_PARAM_INVALID, "a block_table was passed but kv_layout is contiguous");
    } else {
        if (!p->block_table) return fail(FA_ERR_NULLPTR, "a paged kv_layout needs a block_table");
        if (!p->actual_seq_lengths)
            return fail(FA_ERR_NULLPTR, "a paged kv_layout needs actual_seq_lengths");
        if (p->block_size < 16 || p->block_size > 1024 || p->block_size % 16 != 0)
            return fail(FA_ERR_PARAM_INVALID, "block_size must be a multiple of 16 in [16, 1024], got %lld",
                        (long long)p->block_size);
        if (p->max_blocks_per_seq < 1 || p->max_blocks_per_seq >= kMaxDim)
            return fail(FA_ERR_PARAM_INVALID, "max_blocks_per_seq must be in [1, 2^31), got %lld",
                        (long long)p->max_blocks_per_seq);
        if (p->num_blocks < 1 || p->num_blocks >= kMaxDim)
            return fail(FA_ERR_PARAM_INVALID, "num_blocks must be in [1, 2^31), got %lld", (long long)p->num_blocks);
        if (p->kv_seq > p->max_blocks_per_seq * p->block_size)
            return fail(FA_ERR_PARAM_INVALID, "kv_seq (%lld) exceeds max_blocks_per_seq * block_size (%lld)",
                        (long long)p->kv_seq, (long long)(p->max_blocks_per_seq * p->block_size));
        if (p->batch * p->max_blocks_per_seq >= kMaxDim)
            return fail(FA_ERR_PARAM_INVALID, "batch * max_blocks_per_seq must stay below 2^31");
    }
    s->B = p->batch;
    s->QN = p->num_heads;
    s->KVN = kvn;
    s->QS = p->q_seq;
    s->KVS = p->kv_seq;
    s->D = p->head_dim;
    s->g = p->num_heads / kvn;
    if (s->B * s->QN > kMaxDim || s->B * kvn > kMaxDim)
        return fail(FA_ERR_PARAM_INVALID, "batch * heads must stay below 2^31");
    const double qe = (p->layout == FA_TND ? 1.0 : double(s->B)) * double(s->QN) * double(s->QS) * double(s->D);
    const double ke = p->kv_layout == FA_KV_CONTIGUOUS
                          ? (p->layout == FA_TND ? 1.0 : double(s->B)) * double(s->KVN) * double(s->KVS) * double(s->D)
                          : double(p->num_blocks) * double(p->block_size) * double(s->KVN) * double(s->D);
    if (qe >= double(kMaxElems) || ke >= double(kMaxElems)) return fail(FA_ERR_PARAM_INVALID, "tensor too large");
    if (p->kv_layout != FA_KV_CONTIGUOUS && !fast_decode(p) && !general_split_ok(p, *s))
        return fail(FA_ERR_UNSUPPORTED,
                    "a paged KV cache is built for the split-KV paths: one query position without a mask or used "
                    "lengths, or head_dim 64/128 with num_heads / num_kv_heads * q_seq <= 512");
    return ok();
}

fa_status check_tensors(const void* q, const void* k, const void* v, const void* out, const float* lse) {
    if (!q || !k || !v) return fail(FA_ERR_NULLPTR, "q, k and v must not be NULL");
    if (!out) return fail(FA_ERR_NULLPTR, "out must not be NULL");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
        return fail(FA_ERR_PARAM_INVALID, "q, k, v and out must be 16-byte aligned");
    if (lse && !aligned(lse, 4)) return fail(FA_ERR_PARAM_INVALID, "lse must be 4-byte aligned");
    return ok();
}

int heads_per_workgroup(int64_t g) {
    if (g % 8 == 0) return 8;
    if (g % 4 == 0) return 4;
    if (g % 2 == 0) return 2;
    return 1;
}

// Per-device facts the planner needs on every decode call, queried once per
// device (HIP device attribute and occupancy queries cost host time that a
// per-token serving loop should not pay).  Entries are written once with the
// same value by any thread that races to fill them.
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];
// Stage-1 residency per device and (dtype, D, heads per workgroup, paged):
// 2 x 3 x 4 x 2 = 48 instantiations, then the matrix-core stage 1 per
// (dtype, D in {64, 128}, paged, waves); 0 = not asked yet, -1 = no answer.
std::atomic<int> g_resident[kMaxDevices][96];

int current_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
    return dev;
}

int device_cus() {
    const int dev = current_device();
    if (dev < 0) return 256;
    int n = g_cus[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
    g_cus[dev].store(n, std::memory_order_relaxed);
    return n;
}

int stage1_residency(int dtype, int D, int gh, bool paged, bool masked = false) {
    const int dev = current_device();
    const int di = D == 64 ? 0 : (D == 128 ? 1 : 2);
    const int gi = gh == 1 ? 0 : (gh == 2 ? 1 : (gh == 4 ? 2 : 3));
    // keys 0..47 unmasked, 48..63 the matrix-core kernel, 64..87 masked (contiguous)
    const int key = masked ? 64 + (dtype * 3 + di) * 4 + gi : ((dtype * 3 + di) * 4 + gi) * 2 + (paged ? 1 : 0);
    if (dev >= 0) {
        const int cached = g_resident[dev][key].load(std::memory_order_relaxed);
        if (cached != 0) return cached > 0 ? cached : 0;
    }
    const int n = fa::decode_stage1_residency(dtype, D, gh, paged, masked);
    if (dev >= 0) g_resident[dev][key].store(n > 0 ? n : -1, std::memory_order_relaxed);
    return n;
}

int mfma_residency(int dtype, int D, bool paged, int waves) {
    const int dev = current_device();
    const int key = 48 + ((dtype * 2 + (D == 64 ? 0 : 1)) * 2 + (paged ? 1 : 0)) * 2 + (waves == 1 ? 0 : 1);
    if (dev >= 0) {
        const int cached = g_resident[dev][key].load(std::memory_order_relaxed);
        if (cached != 0) return cached > 0 ? cached : 0;
    }
    const int n = fa::decode_mfma_residency(dtype, D, paged, waves);
    if (dev >= 0) g_resident[dev][key].store(n > 0 ? n : -1, std::memory_order_relaxed);
    return n;
}

// Grouped query heads (4 to 32 per KV head) run the matrix-core stage 1: the
// heads of a KV head form the rows of one matrix tile, where the vector-ALU
// stage 1 spends a dot-product reduction and an exponential per head on
// every lane of a row's group and is bound by that vector work rather than
// by HBM.  Its tiles address 64 rows with 32-bit offsets; on a paged cache a
// wave load of 4 or 8 rows stays in one block (block sizes are multiples of
// 16).
int64_t kv_row_bytes(const fa_params* p, const Shape& s) {
    if (p->kv_layout == FA_KV_PAGED_BBND) return s.KVN * s.D * 2;
    if (p->kv_layout == FA_KV_PAGED_BNBD) return s.D * 2;
    return (p->layout == FA_BNSD ? s.D : s.KVN * s.D) * 2;
}
bool mfma_decode(const fa_params* p, const Shape& s) {
    return s.g >= 4 && s.g <= 32 && (s.D == 64 || s.D == 128) && kv_row_bytes(p, s) * 64 < (int64_t(1) << 31) &&
           (p->kv_layout == FA_KV_CONTIGUOUS || p->block_size % 16 == 0);
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Partials {
    size_t o_bytes, m_bytes, c_bytes, total;
};

// Workspace of a split plan: o_part, m_part, l_part (fa_decode_splitkv's
// layouts), then one counter per stage-1 unit for the fused plan.
Partials partial_bytes(const Shape& s, int64_t splits) {
    Partials r;
    const size_t rows = size_t(s.B) * size_t(s.QN) * size_t(s.QS) * size_t(splits);
    r.o_bytes = round_up(rows * size_t(s.D) * sizeof(float), 256);
    r.m_bytes = round_up(rows * sizeof(float), 256);
    const size_t units = size_t(s.B) * size_t(s.KVN) * size_t(s.g / heads_per_workgroup(s.g));
    r.c_bytes = round_up(units * sizeof(unsigned), 256);
    r.total = r.o_bytes + 2 * r.m_bytes + r.c_bytes;
    return r;
}

// Split plan.  Decode reads each KV byte once, so every CU must stream: aim for
// as many stage-1 workgroups as the CUs hold at once (the occupancy of the
// instantiation that will run, four per CU when no device answers), so the
// grid is one full round with no straggling second one.  The units of
// independent work are (b, kv head, head group); when there are fewer than
// that target, the KV axis is cut into chunks (multiples of 64 tokens, at
// least 256) so that units * splits reaches it.  One split means stage 1
// finishes in place.
constexpr int64_t kMinChunk = 256;
constexpr int64_t kWgPerCu = 4;

// Largest chunk: a paged cache's block ids (at most chunk/block_size + 1) must
// fit the stage-1 kernel's LDS table; a contiguous chunk (plus the rows loaded
// ahead of it) must stay addressable with 32-bit byte offsets.
int64_t chunk_cap(const fa_params* p, const Shape& s) {
    if (p->kv_layout != FA_KV_CONTIGUOUS) return (fa::kPagedTableLds - 8) * p->block_size;
    const int64_t row_bytes = (p->layout == FA_BNSD ? s.D : s.KVN * s.D) * 2;
    return ((int64_t(0x7fffffff) / row_bytes - 256) / 64) * 64;
}

// The matrix-core stage 1 runs one wave per workgroup for chunks of at most
// kShortChunk tokens (a few tiles: the time is load latency, and smaller
// workgroups keep more loads in flight per CU) and two waves otherwise.
constexpr int64_t kShortChunk = 512;
int mfma_waves(int64_t chunk) { return chunk <= kShortChunk ? 1 : 2; }
// A one-wave workgroup keeps a paged chunk's block ids in a register.
static_assert(kShortChunk / 16 + 2 <= fa::kLaneBlocks, "one-wave paged chunks outgrow the block-id register");

// Stage 1 runs on the matrix cores: grouped heads on the fast decode path,
// and always on the general split path.
bool uses_mfma(const fa_params* p, const Shape& s) {
    return (fast_decode(p) || vector_masked_decode(p, s)) ? mfma_decode(p, s) : true;
}

void plan_splits(const fa_params* p, const Shape& s, int num_cus, int64_t* splits, int64_t* chunk, int waves = 2) {
    const int gh = heads_per_workgroup(s.g);
    const bool mm = uses_mfma(p, s);
    const bool paged = p->kv_layout != FA_KV_CONTIGUOUS;
    // Units of independent work: (b, KV head) and, on the general path, its
    // row groups.
    const int64_t units = mm ? s.B * s.KVN * (fast_decode(p) ? 1 : row_groups(s)) : s.B * s.KVN * (s.g / gh);
    const int resident = mm ? mfma_residency(p->dtype == FA_BF16 ? 1 : 0, (int)s.D, paged, waves)
                            : stage1_residency(p->dtype == FA_BF16 ? 1 : 0, (int)s.D, gh, paged,
                                               vector_masked_decode(p, s));
    const int64_t cus = num_cus > 0 ? num_cus : 256;
    int64_t per_cu = resident > 0 ? resident : kWgPerCu;
    // The vector stage 1 on a cache whose rows of one head are contiguous
    // (BNSD, or paged with blocks per head) streams best at four workgroups per
    // CU (measured on MI355X: 1.6-2.2 % faster than at the five that fit) when
    // its units divide that many evenly; an uneven split leaves some CUs a
    // fifth workgroup that sets the time, so the planner then fills what fits.
    // (BSND caches measured either way between runs: they keep what fits.)
    const bool head_rows = p->kv_layout == FA_KV_PAGED_BNBD || (p->kv_layout == FA_KV_CONTIGUOUS && p->layout == FA_BNSD);
    if (!mm && head_rows && per_cu > kWgPerCu && (kWgPerCu * cus) % units == 0) per_cu = kWgPerCu;
    const int64_t target = per_cu * cus;
    int64_t want = (target + units - 1) / units;
    if (want < 1) want = 1;
    int64_t c = (s.KVS + want - 1) / want;
    c = (c + 63) / 64 * 64;
    const int64_t kv_round = (s.KVS + 63) / 64 * 64;
    if (c < kMinChunk) c = kMinChunk < kv_round ? kMinChunk : kv_round;
    if (c > chunk_cap(p, s)) c = chunk_cap(p, s);
    *chunk = c;
    *splits = (s.KVS + c - 1) / c;
    // Short chunks: plan again for the one-wave workgroups (more of them fit).
    if (mm && waves == 2 && *splits > 1 && mfma_waves(c) == 1) plan_splits(p, s, num_cus, splits, chunk, 1);
}

// The plan fa_fwd runs for q_seq == 1.  With per-batch lengths the
// matrix-core stage 1 takes a length-balanced schedule instead of fixed
// chunks: the lengths live on the device, so the kernels derive the pieces
// from them (bal_locate), every piece about the same work, none empty; the
// host sizes the launch (target + B * KV_N workgroups) and the partials
// (slots per row: at most ceil(kv_seq / 64) and ceil(target / KV_N) + 1).
struct DecodePlan {
    int64_t splits;  // fixed plan: chunks; balanced plan: slots per row
    int64_t chunk;
    int32_t bal_nwg; // 0 = fixed plan
    int waves;       // matrix-core stage 1: waves per workgroup
};
// Balanced plan for a wave count; false when a paged piece could outgrow the
// on-chip block table.
bool balanced_plan(const fa_params* p, const Shape& s, int waves, DecodePlan* d) {
    const bool paged = p->kv_layout != FA_KV_CONTIGUOUS;
    const int res = mfma_residency(p->dtype == FA_BF16 ? 1 : 0, (int)s.D, paged, waves);
    const int64_t slots = int64_t(res > 0 ? res : 2) * device_cus();
    // Rounding each batch's pieces up adds at most one piece per (batch,
    // KV head): aim at slots - B*KV_N pieces so the whole grid (target +
    // B*KV_N workgroups) fits in the resident slots and runs as one round.
    const int64_t units = s.B * s.KVN;
    const int64_t nwg = slots - units > (slots + 1) / 2 ? slots - units : (slots + 1) / 2;
    const int64_t by_len = (s.KVS + 63) / 64;
    const int64_t by_wg = (nwg + s.KVN - 1) / s.KVN + 1;
    // A paged piece's block ids are staged on chip: bound the largest
    // piece (every batch at full length) by the table.
    const int64_t tmax = (s.KVN * s.B * by_len + nwg - 1) / nwg;
    const int64_t table = waves == 1 ? fa::kLaneBlocks : fa::kPagedTableLds;
    if (paged && tmax * 64 / p->block_size + 2 > table) return false;
    d->bal_nwg = (int32_t)nwg;
    d->splits = by_len < by_wg ? by_len : by_wg;
    d->chunk = 64;
    d->waves = waves;
    return true;
}
DecodePlan decode_plan(const fa_params* p, const Shape& s) {
    DecodePlan d;
    plan_splits(p, s, device_cus(), &d.splits, &d.chunk);
    d.bal_nwg = 0;
    d.waves = mfma_waves(d.chunk);
    if (fast_decode(p) && mfma_decode(p, s) && p->actual_seq_lengths && d.splits > 1) {
        // The balanced pieces share out what the fixed chunks would cover at
        // full lengths, so they are no longer: the fixed plan's wave count holds.
        DecodePlan b = d;
        if (balanced_plan(p, s, d.waves, &b)) d = b;
    }
    return d;
}

// One query position, no mask, no used lengths: the decode kernels of
// stage 1 (vector or matrix-core) with fixed or length-balanced pieces.
bool fast_decode(const fa_params* p) {
    return p->q_seq == 1 && p->mask_mode == FA_MASK_NONE && !p->seqused_q && p->layout != FA_TND;
}

// One query position under a boolean mask tensor with unit key stride, on a
// contiguous cache, in
// a shape the matrix-core stage 1 does not take (fewer than 4 or more than 32
// query heads per KV head, or head_dim 256): the vector stage 1 applies the
// mask per key (aclnnIncreFlashAttention, attenMask of shape (B|1, N|1, 1, S))
// and the split plan is the unmasked one.
bool vector_masked_decode(const fa_params* p, const Shape& s) {
    return p->q_seq == 1 && p->mask_mode == FA_MASK_BOOL && p->mask_stride[3] == 1 && !p->seqused_q &&
           p->layout != FA_TND && p->kv_layout == FA_KV_CONTIGUOUS && !mfma_decode(p, s);
}

// The split-KV stage 1 on the matrix cores in its general form: the g * Q_S
// (query head, position) rows of a KV head fill up to sixteen 32-row tiles,
// masks (causal, window, boolean tensor) and used lengths applied per key,
// and the combine merges the pieces (FlashAttn developer guide 1.9 and 4:
// FlashDecode splits the KV axis when the query rows alone cannot occupy the
// cores, e.g. S1 = 1).
constexpr int64_t kMaxSplitRows = 512;
bool general_split_ok(const fa_params* p, const Shape& s) {
    return p->layout != FA_TND && (s.D == 64 || s.D == 128) && s.g * s.QS <= kMaxSplitRows &&
           kv_row_bytes(p, s) * 64 < (int64_t(1) << 31) &&
           (p->kv_layout == FA_KV_CONTIGUOUS || p->block_size % 16 == 0);
}
int row_groups(const Shape& s) { return (int)((s.g * s.QS + 31) / 32); }

// Prefill workgroups for this shape: the interleaved kernel's tiles (256
// rows at D = 128, 128 at D = 256), 128-row tiles for the tiled kernel.
int64_t prefill_workgroups(const fa_params* p, const Shape& s) {
    const int64_t rows = fa::prefill_rows_per_tile((int)s.D, prefill_mask_kind(p, s), mask_in_dwords(p, s));
    return s.B * s.QN * ((s.QS + rows - 1) / rows);
}

// Keys a query row can see at most: the causal mask is top-left (row i sees
// keys j <= i), the window reaches win_right past the row.
int64_t visible_keys(const fa_params* p, const Shape& s) {
    int64_t n = s.KVS;
    if (p->mask_mode == FA_MASK_CAUSAL && n > s.QS) n = s.QS;
    // (compared as n - Q_S > win_right: win_right may be as large as int64 allows)
    if (p->mask_mode == FA_MASK_WINDOW && p->win_right >= 0 && n - s.QS > p->win_right) n = s.QS + p->win_right;
    return n;
}
// Below this many visible keys the split's extra launch and merge cost more
// than the idle CUs of a small prefill grid.  Measured on MI355X with small
// grids (8 to 32 prefill workgroups): a prefill costs about 1.2 us per 64
// keys at head_dim 128 and 0.8 us at 64 over a fixed ~8 us, the split
// 14-19 us whatever the length; the two cross between 512 and 768 keys at
// head_dim 128 (Q_S = 64: 17.1 against 17.7 us at 512, 21.7 against 17.9 at
// 768) and near 1024 at head_dim 64 (19.0 against 19.3 us).
int64_t split_min_keys(const Shape& s) { return s.D >= 128 ? 640 : 1024; }

enum class Path { kPrefill, kFastDecode, kSplit };
Path choose_path(const fa_params* p, const Shape& s) {
    if (p->layout == FA_TND) return Path::kPrefill;
    if (fast_decode(p) || vector_masked_decode(p, s)) return Path::kFastDecode;
    if (!general_split_ok(p, s)) return Path::kPrefill;
    // One query position always splits (masked decode); a few positions split
    // when the prefill's query tiles cannot fill the CUs and the rows see
    // enough keys to pay for the split.
    if (s.QS == 1 || p->kv_layout != FA_KV_CONTIGUOUS) return Path::kSplit;
    return (prefill_workgroups(p, s) < device_cus() && visible_keys(p, s) >= split_min_keys(s)) ? Path::kSplit
                                                                                          : Path::kPrefill;
}
bool decode_path(const fa_params* p) { return fast_decode(p); }

// Packed layout: entries of the cost-ordered work list, one per 128-row query
// tile of every sequence plus the rows past the last sequence.  The sum over
// the B + 1 sequences of ceil(rows / 128) is at most ceil(Q_T / 128) + B + 1.
int64_t varlen_capacity(const Shape& s) { return (s.QS + 127) / 128 + s.B + 1; }
size_t varlen_bytes(const Shape& s) { return round_up(size_t(varlen_capacity(s)) * 8, 256); }

// Prefill kernel instantiation for the mask: 0 none, 1 causal, 2 boolean
// tensor read element by element, 3 boolean tensor staged through LDS (rows
// of contiguous, 16-byte aligned key runs), 4 window.
// A boolean tensor whose rows are runs of 4-byte aligned keys (unit key
// stride, strides and kv_seq multiples of 4, row offsets within 32 bits): the
// interleaved prefill stages it with 4-byte loads.
bool mask_in_dwords(const fa_params* p, const Shape& s) {
    const int64_t* st = p->mask_stride;
    return p->mask_mode == FA_MASK_BOOL && aligned(p->mask, 4) && st[3] == 1 && st[0] >= 0 && st[1] >= 0 &&
           st[2] >= 0 && st[0] % 4 == 0 && st[1] % 4 == 0 && st[2] % 4 == 0 && s.KVS % 4 == 0 &&
           st[2] < (int64_t(1) << 28);
}

int prefill_mask_kind(const fa_params* p, const Shape& s) {
    if (p->mask_mode == FA_MASK_CAUSAL) return 1;
    if (p->mask_mode == FA_MASK_WINDOW) return 4;
    if (p->mask_mode != FA_MASK_BOOL) return 0;
    const int64_t* st = p->mask_stride;
    const bool rows_ok = st[3] == 1 && aligned(p->mask, 16) && st[0] % 16 == 0 && st[1] % 16 == 0 &&
                         st[2] % 16 == 0 && s.KVS % 16 == 0 && st[2] < (int64_t(1) << 23);
    return rows_ok ? 3 : 2;
}

// Staged boolean mask: geometry of its per-tile summary (one row of words
// per mask slice and 128-row query tile).  blocks == 0 when the mask is not
// staged, or the summary would need more than 2^31 - 1 workgroups.
struct MaskSummaryGeom {
    int64_t q_tiles, words, slices_n, blocks;
    size_t bytes;
};
MaskSummaryGeom mask_summary_geom(const fa_params* p, const Shape& s) {
    MaskSummaryGeom g{0, 0, 0, 0, 0};
    if (p->layout == FA_TND || choose_path(p, s) != Path::kPrefill || prefill_mask_kind(p, s) != 3) return g;
    const int64_t kv_tiles = (s.KVS + fa::kMaskKeysPerTile - 1) / fa::kMaskKeysPerTile;
    g.q_tiles = (s.QS + fa::kMaskRowsPerTile - 1) / fa::kMaskRowsPerTile;
    g.words = (kv_tiles + fa::kMaskTilesPerWord - 1) / fa::kMaskTilesPerWord;
    g.slices_n = p->mask_stride[1] ? s.QN : 1;
    const int64_t slices = (p->mask_stride[0] ? s.B : 1) * g.slices_n;
    const double blocks = double(slices) * double(g.q_tiles) * double(g.words);
    if (blocks > double(0x7fffffff)) return MaskSummaryGeom{0, 0, 0, 0, 0};
    g.blocks = slices * g.q_tiles * g.words;
    g.bytes = round_up(size_t(g.blocks) * 4, 256);
    return g;
}

void fill_decode_args(const fa_params* p, const Shape& s, fa::DecodeArgs* a) {
    std::memset(a, 0, sizeof *a);
    a->lens = p->actual_seq_lengths;
    a->kv_seq = s.KVS;
    if (p->kv_layout == FA_KV_PAGED_BBND) {
        a->kv_stride_s = s.KVN * s.D;
        a->kv_stride_n = s.D;
        a->kv_stride_blk = p->block_size * s.KVN * s.D;
    } else if (p->kv_layout == FA_KV_PAGED_BNBD) {
        a->kv_stride_s = s.D;
        a->kv_stride_n = p->block_size * s.D;
        a->kv_stride_blk = s.KVN * p->block_size * s.D;
    } else if (p->layout == FA_BNSD) {
        a->kv_stride_s = s.D;
        a->kv_stride_n = s.KVS * s.D;
        a->kv_stride_b = s.KVN * s.KVS * s.D;
    } else {
        a->kv_stride_s = s.KVN * s.D;
        a->kv_stride_n = s.D;
        a->kv_stride_b = s.KVS * s.KVN * s.D;
    }
    if (p->kv_layout != FA_KV_CONTIGUOUS) {
        a->block_table = p->block_table;
        a->block_size = (int32_t)p->block_size;
        a->max_blocks = (int32_t)p->max_blocks_per_seq;
        a->num_blocks = (int32_t)p->num_blocks;
    }
    a->num_heads = (int32_t)s.QN;
    a->num_kv_heads = (int32_t)s.KVN;
    a->group = (int32_t)s.g;
    const int gh = heads_per_workgroup(s.g);
    a->head_groups = (int32_t)(s.g / gh);
    a->scale_log2 = (float)(p->scale * 1.4426950408889634);
    if (a->scale_log2 == 0.f) {  // scale 0 (or below fp32's range): every score is 0
        a->zero_q = 1;
        a->scale_log2 = 1.f;
    }
    a->batch = (int32_t)s.B;
    a->q_seq = s.QS;
    a->q_stride_b = s.QS * s.QN * s.D;
    a->q_stride_n = p->layout == FA_BNSD ? s.QS * s.D : s.D;
    a->q_stride_s = p->layout == FA_BNSD ? s.D : s.QN * s.D;
    a->out_bsnd = p->layout == FA_BSND ? 1 : 0;
    a->row_groups = fast_decode(p) ? 1 : row_groups(s);
    a->used_q = p->seqused_q;
    a->mask_mode = (int32_t)p->mask_mode;  // 1 causal, 2 boolean tensor, 3 window
    if (p->mask_mode == FA_MASK_BOOL) {
        a->mask = p->mask;
        for (int i = 0; i < 4; ++i) a->mask_stride[i] = p->mask_stride[i];
        const int64_t* st = p->mask_stride;
        a->mask_dword = (aligned(p->mask, 4) && st[3] == 1 && st[0] % 4 == 0 && st[1] % 4 == 0 && st[2] % 4 == 0 &&
                         s.KVS % 4 == 0)
                            ? 1
                            : 0;
    }
    auto win = [](int64_t w) { return (w < 0 || w > 0x7fffffff) ? int32_t(0x7fffffff) : int32_t(w); };
    a->win_left = win(p->win_left);
    a->win_right = win(p->win_right);
}

fa_status launch_result(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(FA_ERR_RUNTIME, "%s launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

fa_status run_stage1(const fa_params* p, const Shape& s, int64_t splits, int64_t chunk, const void* q, const void* k,
                     const void* v, float* o_part, float* m_part, float* l_part, unsigned* counters, void* out,
                     float* lse, hipStream_t stream, int32_t bal_nwg = 0, int waves = 0) {
    fa::DecodeArgs a;
    fill_decode_args(p, s, &a);
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.o_part = o_part;
    a.m_part = m_part;
    a.l_part = l_part;
    a.out = out;
    a.lse = lse;
    a.chunk = chunk;
    a.num_splits = (int32_t)splits;
    a.counters = counters;
    a.bal_nwg = bal_nwg;
    const bool finish = (out != nullptr && counters == nullptr);
    if (counters == nullptr && uses_mfma(p, s))
        return launch_result(fa::launch_decode_mfma(a, p->dtype == FA_BF16 ? 1 : 0, (int)s.D, finish,
                                                    waves > 0 ? waves : mfma_waves(chunk), s.B, stream),
                             "decode stage 1");
    return launch_result(fa::launch_decode_stage1(a, p->dtype == FA_BF16 ? 1 : 0, (int)s.D,
                                                  heads_per_workgroup(s.g), finish, s.B, stream),
                         "decode stage 1");
}

fa_status run_combine(const fa_params* p, const Shape& s, int64_t splits, const float* o_part, const float* m_part,
                      const float* l_part, void* out, float* lse, hipStream_t stream, int32_t bal_nwg = 0) {
    fa::CombineArgs a;
    std::memset(&a, 0, sizeof a);
    a.bal_nwg = bal_nwg;
    a.lens = p->actual_seq_lengths;
    a.kv_seq = s.KVS;
    a.batch = (int32_t)s.B;
    a.num_heads = (int32_t)s.QN;
    a.num_kv_heads = (int32_t)s.KVN;
    a.o_part = o_part;
    a.m_part = m_part;
    a.l_part = l_part;
    a.out = out;
    a.lse = lse;
    a.rows = s.B * s.QN * s.QS;
    a.q_seq = s.QS;
    a.out_bsnd = p->layout == FA_BSND ? 1 : 0;
    a.num_splits = (int32_t)splits;
    return launch_result(fa::launch_combine(a, p->dtype == FA_BF16 ? 1 : 0, (int)s.D, stream), "combine");
}

fa_status run_prefill(const fa_params* p, const Shape& s, const void* q, const void* k, const void* v, void* out,
                      float* lse, void* workspace, hipStream_t stream) {
    // The prefill kernel addresses one 64-row KV tile with 32-bit byte offsets.
    const int64_t kv_row_elems = p->layout == FA_BNSD ? s.D : s.KVN * s.D;
    if (kv_row_elems * 2 * 64 >= (int64_t(1) << 31))
        return fail(FA_ERR_UNSUPPORTED, "prefill needs num_kv_heads * head_dim < 2^24 in the BSND layout");
    fa::PrefillArgs a;
    std::memset(&a, 0, sizeof a);
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.out = out;
    a.lse = lse;
    a.lens = p->actual_seq_lengths;
    a.mask = p->mask;
    for (int i = 0; i < 4; ++i) a.mask_stride[i] = p->mask_stride[i];
    a.q_seq = s.QS;
    a.kv_seq = s.KVS;
    if (p->layout == FA_BNSD) {
        a.q_stride_s = s.D;
        a.q_stride_n = s.QS * s.D;
        a.q_stride_b = s.QN * s.QS * s.D;
        a.kv_stride_s = s.D;
        a.kv_stride_n = s.KVS * s.D;
        a.kv_stride_b = s.KVN * s.KVS * s.D;
    } else {
        a.q_stride_s = s.QN * s.D;
        a.q_stride_n = s.D;
        a.q_stride_b = s.QS * s.QN * s.D;
        a.kv_stride_s = s.KVN * s.D;
        a.kv_stride_n = s.D;
        a.kv_stride_b = s.KVS * s.KVN * s.D;
    }
    if (p->layout == FA_TND) {  // [T][N][D]: rows of a sequence are BSND rows
        a.q_stride_s = s.QN * s.D;
        a.q_stride_n = s.D;
        a.q_stride_b = 0;
        a.kv_stride_s = s.KVN * s.D;
        a.kv_stride_n = s.D;
        a.kv_stride_b = 0;
    }
    a.num_heads = (int32_t)s.QN;
    a.num_kv_heads = (int32_t)s.KVN;
    a.group = (int32_t)s.g;
    a.q_tiles = (int32_t)((s.QS + 127) / 128);
    a.negate_q = p->scale < 0 ? 1 : 0;
    a.scale_log2 = (float)(std::fabs(p->scale) * 1.4426950408889634);
    if (a.scale_log2 == 0.f) {  // scale 0 (or below fp32's range): every score is 0
        a.zero_q = 1;
        a.scale_log2 = 1.f;
    }
    a.used_q = p->seqused_q;  // padded layouts: rows past it written as 0 / +inf
    // Window bounds as 32-bit distances from the query row: |key - row| < 2^31.
    auto win = [](int64_t w) { return (w < 0 || w > 0x7fffffff) ? int32_t(0x7fffffff) : int32_t(w); };
    a.win_left = win(p->win_left);
    a.win_right = win(p->win_right);
    const int mm = prefill_mask_kind(p, s);
    a.mask_dwords = mask_in_dwords(p, s) ? 1 : 0;
    // A staged boolean mask with a workspace is summarised per tile first, so
    // the prefill skips the tiles it masks entirely and the mask loads of
    // tiles it does not mask at all.
    const MaskSummaryGeom mg = mask_summary_geom(p, s);
    if (mg.blocks > 0 && workspace) {
        fa::MaskSummaryArgs ma;
        std::memset(&ma, 0, sizeof ma);
        ma.mask = p->mask;
        for (int i = 0; i < 4; ++i) ma.mask_stride[i] = p->mask_stride[i];
        ma.q_seq = s.QS;
        ma.kv_seq = s.KVS;
        ma.q_tiles = (int32_t)mg.q_tiles;
        ma.words = (int32_t)mg.words;
        ma.slices_n = (int32_t)mg.slices_n;
        ma.blocks = mg.blocks;
        ma.out = static_cast<uint32_t*>(workspace);
        fa_status st = launch_result(fa::launch_mask_summary(ma, stream), "mask summary");
        if (st != FA_OK) return st;
        a.mask_cls = ma.out;
        a.cls_words = ma.words;
    }
    if (p->layout == FA_TND) {
        fa::VarlenScheduleArgs sa;
        std::memset(&sa, 0, sizeof sa);
        sa.cu_q = p->cu_seqlens_q;
        sa.cu_kv = p->cu_seqlens_kv;
        sa.used_q = p->seqused_q;
        sa.lens = p->actual_seq_lengths;
        sa.work = static_cast<int32_t*>(workspace);
        sa.q_total = s.QS;
        sa.kv_total = s.KVS;
        sa.batch = (int32_t)s.B;
        sa.capacity = (int32_t)varlen_capacity(s);
        sa.mask_mode = mm;
        sa.win_left = a.win_left;
        sa.win_right = a.win_right;
        sa.rows = fa::prefill_rows_per_tile((int)s.D, mm, a.mask_dwords != 0);
        fa_status st = launch_result(fa::launch_varlen_schedule(sa, stream), "packed-batch schedule");
        if (st != FA_OK) return st;
        a.cu_q = p->cu_seqlens_q;
        a.cu_kv = p->cu_seqlens_kv;
        a.used_q = p->seqused_q;
        a.work = sa.work;
        a.work_items = sa.capacity;
        a.batch = (int32_t)s.B;
    }
    a.cus = device_cus();
    return launch_result(fa::launch_prefill(a, p->dtype == FA_BF16 ? 1 : 0, (int)s.D, mm, s.B, stream), "prefill");
}

// The split-KV entry points: the fast decode shape (one position, no mask,
// no used lengths: any head_dim) or the general matrix-core shape.
fa_status check_split_shape(const fa_params* p, const Shape& s) {
    if (p->layout == FA_TND) return fail(FA_ERR_UNSUPPORTED, "split-KV decode is built for BNSD and BSND");
    if (fast_decode(p) || vector_masked_decode(p, s) || general_split_ok(p, s)) return ok();
    return fail(FA_ERR_UNSUPPORTED,
                "split-KV with several query positions, a mask or used lengths is built for head_dim 64 and 128 "
                "with num_heads / num_kv_heads * q_seq <= %lld",
                (long long)kMaxSplitRows);
}

// Scratch of fa_fwd_noalloc: device memory the library holds itself, so that
// callers that cannot allocate (code under HIP graph capture, serving loops,
// harnesses that forbid it) still run the paths that need a workspace.  One
// copy per GPU, resident from the module's load until the process ends.  In
// host code `scratch` only names the symbol: its device address comes from
// hipGetSymbolAddress, asked once per device with that device current.
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Device address of this device's scratch, or nullptr (with the error set).
void* scratch_address(int dev) {
    void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (ptr) return ptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
        fail(FA_ERR_RUNTIME, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
        return nullptr;
    }
    g_scratch_ptr[dev].store(ptr, std::memory_order_release);
    return ptr;
}

// One line naming what fa_fwd launches for p: the path, each kernel with its
// instantiation and grid, the split plan and the workspace it needs.
std::string describe(const fa_params* p, const Shape& s) {
    static const char* kMask[] = {"none", "causal", "bool", "window"};
    const char* dt = p->dtype == FA_BF16 ? "BF16" : "F16";
    const char* lay = p->layout == FA_TND ? "TND" : (p->layout == FA_BSND ? "BSND" : "BNSD");
    const char* kv = p->kv_layout == FA_KV_PAGED_BBND ? "PA_BBND" : (p->kv_layout == FA_KV_PAGED_BNBD ? "PA_BNBD" : "contiguous");
    const int mmode = (p->mask_mode >= 0 && p->mask_mode <= 3) ? (int)p->mask_mode : 0;
    char head[256], body[512];
    std::snprintf(head, sizeof head, "%s %s B=%lld Q_N=%lld KV_N=%lld Q_S=%lld KV_S=%lld D=%lld mask=%s kv=%s", lay, dt,
                  (long long)s.B, (long long)s.QN, (long long)s.KVN, (long long)s.QS, (long long)s.KVS, (long long)s.D,
                  kMask[mmode], kv);
    size_t ws = 0;
    if (p->layout == FA_TND) {
        ws = varlen_bytes(s);
    } else if (choose_path(p, s) == Path::kPrefill) {
        ws = mask_summary_geom(p, s).bytes;
    } else {
        const DecodePlan dp = decode_plan(p, s);
        if (dp.splits > 1 || dp.bal_nwg > 0) ws = partial_bytes(s, dp.splits).total;
    }
    const Path path = choose_path(p, s);
    if (path == Path::kPrefill) {
        const int mk = prefill_mask_kind(p, s);
        const bool dw = mask_in_dwords(p, s);
        const bool il = fa::prefill_interleaved((int)s.D, mk, dw);
        const int64_t rows = fa::prefill_rows_per_tile((int)s.D, mk, dw);
        const MaskSummaryGeom mg = mask_summary_geom(p, s);
        char grid[160];
        const int64_t units =
            p->layout == FA_TND ? (varlen_capacity(s) + 7) / 8 * 8 * s.QN : prefill_workgroups(p, s);
        const int64_t pg = il ? fa::prefill_persistent_grid((int)s.D, mk, units, device_cus()) : 0;
        if (p->layout == FA_TND && pg)
            std::snprintf(grid, sizeof grid, "%lld (persistent, over the work list of <= %lld items x %lld heads)",
                          (long long)pg, (long long)varlen_capacity(s), (long long)s.QN);
        else if (p->layout == FA_TND)
            std::snprintf(grid, sizeof grid, "(work list of <= %lld items) x %lld heads", (long long)varlen_capacity(s),
                          (long long)s.QN);
        else if (pg)
            std::snprintf(grid, sizeof grid, "%lld (persistent, over %lld units)", (long long)pg, (long long)units);
        else
            std::snprintf(grid, sizeof grid, "%lld", (long long)units);
        std::snprintf(body, sizeof body, "path=prefill%s%s kernel=%s<%s,%lld,%d> rows=%lld workgroups=%s%s",
                      p->layout == FA_TND ? " pre=varlen_schedule_kernel" : "",
                      mg.blocks > 0 ? " pre=mask_summary_kernel (with a workspace)" : "",
                      il ? "prefill_il_kernel" : "prefill_kernel", dt, (long long)s.D, mk, (long long)rows, grid,
                      mk == 2 ? (dw ? " mask=4-byte runs" : " mask=element-wise") : "");
    } else {
        const DecodePlan dp = decode_plan(p, s);
        const bool mm = uses_mfma(p, s);
        const bool split = dp.splits > 1 || dp.bal_nwg > 0;
        char plan[128];
        if (dp.bal_nwg > 0)
            std::snprintf(plan, sizeof plan, "length-balanced pieces=%d slots/row=%lld", dp.bal_nwg, (long long)dp.splits);
        else
            std::snprintf(plan, sizeof plan, "splits=%lld chunk=%lld", (long long)dp.splits, (long long)dp.chunk);
        std::snprintf(body, sizeof body, "path=%s stage1=%s%s%s %s%s", path == Path::kFastDecode ? "decode" : "general-split",
                      mm ? "decode_mfma_kernel waves=" : "decode_stage1_kernel", mm ? std::to_string(dp.waves).c_str() : "",
                      (!mm && p->mask_mode == FA_MASK_BOOL) ? " (masked)" : "", plan,
                      split ? " then combine_kernel" : " (finishes in place)");
    }
    char line[900];
    std::snprintf(line, sizeof line, "%s -> %s workspace=%zu", head, body, ws);
    return line;
}

bool log_enabled() {
    static const bool on = [] {
        const char* e = std::getenv("FA_LOG");
        return e && e[0] && std::strcmp(e, "0") != 0;
    }();
    return on;
}

}  // namespace

extern "C" {

const char* fa_last_error(void) { return g_last_error.c_str(); }

fa_status fa_describe(const fa_params* p, char* buf, size_t buf_bytes) {
    Shape s;
    fa_status st = check_params(p, &s);
    if (st != FA_OK) return st;
    if (!buf || buf_bytes == 0) return fail(FA_ERR_NULLPTR, "buf must not be NULL and buf_bytes must be > 0");
    const std::string d = describe(p, s);
    std::snprintf(buf, buf_bytes, "%s", d.c_str());
    return ok();
}

fa_status fa_splitkv_plan(const fa_params* p, int num_cus, int64_t chunk_hint, int64_t* num_splits, int64_t* chunk,
                          size_t* workspace_bytes) {
    Shape s;
    fa_status st = check_params(p, &s);
    if (st != FA_OK) return st;
    if (!num_splits || !chunk) return fail(FA_ERR_NULLPTR, "num_splits and chunk outputs must not be NULL");
    st = check_split_shape(p, s);
    if (st != FA_OK) return st;
    if (chunk_hint < 0 || chunk_hint % 64 != 0)
        return fail(FA_ERR_PARAM_INVALID, "chunk_hint must be 0 or a positive multiple of 64, got %lld",
                    (long long)chunk_hint);
    if (chunk_hint > chunk_cap(p, s))
        return fail(FA_ERR_PARAM_INVALID, "chunk_hint %lld exceeds the largest chunk, %lld tokens",
                    (long long)chunk_hint, (long long)chunk_cap(p, s));
    int64_t sp, c;
    if (chunk_hint > 0) {
        c = chunk_hint;
        sp = (s.KVS + c - 1) / c;
    } else {
        plan_splits(p, s, num_cus > 0 ? num_cus : device_cus(), &sp, &c);
    }
    if (sp > kMaxSplits) return fail(FA_ERR_PARAM_INVALID, "plan needs %lld splits (max %lld)", (long long)sp, (long long)kMaxSplits);
    *num_splits = sp;
    *chunk = c;
    if (workspace_bytes) *workspace_bytes = partial_bytes(s, sp).total;
    return ok();
}

fa_status fa_decode_fused_plan(const fa_params* p, int num_cus, int64_t* num_splits, int64_t* chunk,
                               size_t* workspace_bytes) {
    Shape s;
    fa_status st = check_params(p, &s);
    if (st != FA_OK) return st;
    if (!num_splits || !chunk) return fail(FA_ERR_NULLPTR, "num_splits and chunk outputs must not be NULL");
    if (p->layout == FA_TND || !fast_decode(p))
        return fail(FA_ERR_UNSUPPORTED, "the fused decode takes one query position without a mask or used lengths");
    // The fused launch runs the vector stage 1: plan with its residency and
    // its units (b, KV head, head group), at most kFusedMaxSplits pieces.
    const int gh = heads_per_workgroup(s.g);
    const bool paged = p->kv_layout != FA_KV_CONTIGUOUS;
    const int res = stage1_residency(p->dtype == FA_BF16 ? 1 : 0, (int)s.D, gh, paged);
    const int64_t units = s.B * s.KVN * (s.g / gh);
    const int64_t target = (res > 0 ? res : kWgPerCu) * int64_t(num_cus > 0 ? num_cus : device_cus());
    int64_t want = (target + units - 1) / units;
    if (want < 1) want = 1;
    int64_t c = ((s.KVS + want - 1) / want + 63) / 64 * 64;
    const int64_t kv_round = (s.KVS + 63) / 64 * 64;
    if (c < kMinChunk) c = kMinChunk < kv_round ? kMinChunk : kv_round;
    const int64_t c_min = ((s.KVS + fa::kFusedMaxSplits - 1) / fa::kFusedMaxSplits + 63) / 64 * 64;
    if (c < c_min) c = c_min;
    if (c > chunk_cap(p, s)) c = chunk_cap(p, s);
    const int64_t sp = (s.KVS + c - 1) / c;
    if (sp > fa::kFusedMaxSplits)
        return fail(FA_ERR_UNSUPPORTED, "kv_seq %lld needs more than %d pieces of the largest chunk", (long long)s.KVS,
                    fa::kFusedMaxSplits);
    *num_splits = sp;
    *chunk = c;
    if (workspace_bytes) *workspace_bytes = sp > 1 ? partial_bytes(s, sp).total : 0;
    return ok();
}

fa_status fa_workspace_size(const fa_params* p, size_t* bytes) {
    Shape s;
    fa_status st = check_params(p, &s);
    if (st != FA_OK) return st;
    if (!bytes) return fail(FA_ERR_NULLPTR, "bytes output must not be NULL");
    *bytes = 0;
    if (p->layout == FA_TND) {
        *bytes = varlen_bytes(s);
        return ok();
    }
    if (choose_path(p, s) == Path::kPrefill) {
        *bytes = mask_summary_geom(p, s).bytes;
        return ok();
    }
    const DecodePlan dp = decode_plan(p, s);
    if (dp.splits > 1 || dp.bal_nwg > 0) *bytes = partial_bytes(s, dp.splits).total;
    return ok();
}

fa_status fa_fwd(const fa_params* p, const void* q, const void* k, const void* v, void* out, float* lse,
                 void* workspace, size_t workspace_bytes, void* stream) {
    Shape s;
    fa_status st = check_params(p, &s);
    if (st != FA_OK) return st;
    st = check_tensors(q, k, v, out, lse);
    if (st != FA_OK) return st;
    if (log_enabled()) std::fprintf(stderr, "fa_fwd: %s\n", describe(p, s).c_str());
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (p->layout == FA_TND) {
        const size_t need = varlen_bytes(s);
        if (!workspace) return fail(FA_ERR_NULLPTR, "the TND layout needs %zu bytes of workspace (fa_workspace_size)", need);
        if (!aligned(workspace, 256)) return fail(FA_ERR_PARAM_INVALID, "workspace must be 256-byte aligned");
        if (workspace_bytes < need)
            return fail(FA_ERR_PARAM_INVALID, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, need);
    }
    if (choose_path(p, s) == Path::kPrefill) {
        // A staged boolean mask takes an optional workspace for its summary;
        // without one the prefill runs unchanged, visiting every KV tile.
        const size_t need = mask_summary_geom(p, s).bytes;
        if (p->layout != FA_TND && need && workspace) {
            if (!aligned(workspace, 256)) return fail(FA_ERR_PARAM_INVALID, "workspace must be 256-byte aligned");
            if (workspace_bytes < need)
                return fail(FA_ERR_PARAM_INVALID, "workspace too small: %zu bytes given, %zu needed", workspace_bytes,
                            need);
        }
        return run_prefill(p, s, q, k, v, out, lse, p->layout == FA_TND || need ? workspace : nullptr, hs);
    }

    const DecodePlan dp = decode_plan(p, s);
    const int64_t sp = dp.splits, c = dp.chunk;
    if (sp > kMaxSplits) return fail(FA_ERR_PARAM_INVALID, "plan needs too many splits");
    if (sp == 1 && dp.bal_nwg == 0)
        return run_stage1(p, s, 1, c, q, k, v, nullptr, nullptr, nullptr, nullptr, out, lse, hs);
    const Partials pb = partial_bytes(s, sp);
    if (!workspace) return fail(FA_ERR_NULLPTR, "this call needs %zu bytes of workspace (fa_workspace_size)", pb.total);
    if (!aligned(workspace, 256)) return fail(FA_ERR_PARAM_INVALID, "workspace must be 256-byte aligned");
    if (workspace_bytes < pb.total)
        return fail(FA_ERR_PARAM_INVALID, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, pb.total);
    char* w = static_cast<char*>(workspace);
    float* o_part = reinterpret_cast<float*>(w);
    float* m_part = reinterpret_cast<float*>(w + pb.o_bytes);
    float* l_part = reinterpret_cast<float*>(w + pb.o_bytes + pb.m_bytes);
    st = run_stage1(p, s, sp, c, q, k, v, o_part, m_part, l_part, nullptr, nullptr, nullptr, hs, dp.bal_nwg,
                    dp.waves);
    if (st != FA_OK) return st;
    return run_combine(p, s, sp, o_part, m_part, l_part, out, lse, hs, dp.bal_nwg);
}

fa_status fa_decode_splitkv(const fa_params* p, int64_t num_splits, int64_t chunk, const void* q, const void* k,
                            const void* v, float* o_part, float* m_part, float* l_part, void* stream) {
    Shape s;
    fa_status st = check_params(p, &s);
    if (st != FA_OK) return st;
    st = check_split_shape(p, s);
    if (st != FA_OK) return st;
    if (!q || !k || !v) return fail(FA_ERR_NULLPTR, "q, k and v must not be NULL");
    if (!o_part || !m_part || !l_part) return fail(FA_ERR_NULLPTR, "o_part, m_part and l_part must not be NULL");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16))
        return fail(FA_ERR_PARAM_INVALID, "q, k and v must be 16-byte aligned");
    // o_part rows are written and read as 16-byte vectors
    if (!aligned(o_part, 16) || !aligned(m_part, 4) || !aligned(l_part, 4))
        return fail(FA_ERR_PARAM_INVALID, "o_part must be 16-byte aligned, m_part and l_part 4-byte aligned");
    if (num_splits < 1 || num_splits > kMaxSplits) return fail(FA_ERR_PARAM_INVALID, "num_splits must be in [1, 2^20]");
    if (chunk < 64 || chunk % 64 != 0) return fail(FA_ERR_PARAM_INVALID, "chunk must be a positive multiple of 64");
    if (chunk > chunk_cap(p, s))
        return fail(FA_ERR_PARAM_INVALID, "chunk %lld exceeds the largest chunk, %lld tokens", (long long)chunk,
                    (long long)chunk_cap(p, s));
    if (num_splits * chunk < s.KVS)
        return fail(FA_ERR_PARAM_INVALID, "num_splits * chunk (%lld) must cover kv_seq (%lld)",
                    (long long)(num_splits * chunk), (long long)s.KVS);
    return run_stage1(p, s, num_splits, chunk, q, k, v, o_part, m_part, l_part, nullptr, nullptr, nullptr,
                      static_cast<hipStream_t>(stream));
}

fa_status fa_decode_fused(const fa_params* p, int64_t num_splits, int64_t chunk, const void* q, const void* k,
                          const void* v, void* workspace, size_t workspace_bytes, void* out, float* lse, void* stream) {
    Shape s;
    fa_status st = check_params(p, &s);
    if (st != FA_OK) return st;
    if (p->layout == FA_TND) return fail(FA_ERR_UNSUPPORTED, "split-KV decode is built for BNSD and BSND");
    if (!fast_decode(p))
        return fail(FA_ERR_UNSUPPORTED, "the fused decode takes one query position without a mask or used lengths");
    st = check_tensors(q, k, v, out, lse);
    if (st != FA_OK) return st;
    if (num_splits < 1 || num_splits > fa::kFusedMaxSplits)
        return fail(FA_ERR_PARAM_INVALID, "the fused decode takes 1 to %d splits, got %lld", fa::kFusedMaxSplits,
                    (long long)num_splits);
    if (chunk < 64 || chunk % 64 != 0) return fail(FA_ERR_PARAM_INVALID, "chunk must be a positive multiple of 64");
    if (chunk > chunk_cap(p, s))
        return fail(FA_ERR_PARAM_INVALID, "chunk %lld exceeds the largest chunk, %lld tokens", (long long)chunk,
                    (long long)chunk_cap(p, s));
    if (num_splits * chunk < s.KVS)
        return fail(FA_ERR_PARAM_INVALID, "num_splits * chunk (%lld) must cover kv_seq (%lld)",
                    (long long)(num_splits * chunk), (long long)s.KVS);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (num_splits == 1) return run_stage1(p, s, 1, chunk, q, k, v, nullptr, nullptr, nullptr, nullptr, out, lse, hs);
    const Partials pb = partial_bytes(s, num_splits);
    if (!workspace) return fail(FA_ERR_NULLPTR, "the fused decode needs %zu bytes of workspace", pb.total);
    if (!aligned(workspace, 256)) return fail(FA_ERR_PARAM_INVALID, "workspace must be 256-byte aligned");
    if (workspace_bytes < pb.total)
        return fail(FA_ERR_PARAM_INVALID, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, pb.total);
    char* w = static_cast<char*>(workspace);
    return run_stage1(p, s, num_splits, chunk, q, k, v, reinterpret_cast<float*>(w),
                      reinterpret_cast<float*>(w + pb.o_bytes), reinterpret_cast<float*>(w + pb.o_bytes + pb.m_bytes),
                      reinterpret_cast<unsigned*>(w + pb.o_bytes + 2 * pb.m_bytes), out, lse, hs);
}

fa_status fa_combine(const fa_params* p, int64_t num_splits, const float* o_part, const float* m_part,
                     const float* l_part, void* out, float* lse, void* stream) {
    Shape s;
    fa_status st = check_params(p, &s);
    if (st != FA_OK) return st;
    if (p->layout == FA_TND) return fail(FA_ERR_UNSUPPORTED, "combine is built for BNSD and BSND");
    if (!o_part || !m_part || !l_part) return fail(FA_ERR_NULLPTR, "o_part, m_part and l_part must not be NULL");
    if (!aligned(o_part, 16) || !aligned(m_part, 4) || !aligned(l_part, 4))  // o_part read as 16-byte vectors
        return fail(FA_ERR_PARAM_INVALID, "o_part must be 16-byte aligned, m_part and l_part 4-byte aligned");
    if (!out) return fail(FA_ERR_NULLPTR, "out must not be NULL");
    if (!aligned(out, 16)) return fail(FA_ERR_PARAM_INVALID, "out must be 16-byte aligned");
    if (lse && !aligned(lse, 4)) return fail(FA_ERR_PARAM_INVALID, "lse must be 4-byte aligned");
    if (num_splits < 1 || num_splits > kMaxSplits) return fail(FA_ERR_PARAM_INVALID, "num_splits must be in [1, 2^20]");
    return run_combine(p, s, num_splits, o_part, m_part, l_part, out, lse, static_cast<hipStream_t>(stream));
}

fa_status fa_fwd_noalloc(const fa_params* p, const void* q, const void* k, const void* v, void* out, float* lse,
                         void* stream) {
    size_t need = 0;
    fa_status st = fa_workspace_size(p, &need);
    if (st != FA_OK) return st;
    if (need > kNoallocScratchBytes)
        return fail(FA_ERR_PARAM_INVALID,
                    "fa_fwd_noalloc: this call needs %zu bytes of scratch, the library holds %zu; use fa_fwd with a "
                    "workspace",
                    need, kNoallocScratchBytes);
    void* ws = nullptr;
    if (need > 0) {
        const int dev = current_device();
        if (dev < 0) return fail(FA_ERR_RUNTIME, "fa_fwd_noalloc: no current HIP device");
        ws = scratch_address(dev);
        if (!ws) return FA_ERR_RUNTIME;
    }
    return fa_fwd(p, q, k, v, out, lse, ws, ws ? kNoallocScratchBytes : 0, stream);
}

}  // extern "C"
