// C ABI of libssd: argument checks, planning and the launch sequence.
// Every check runs on the host before anything is launched.
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "../../include/ssd.h"
#include "ssd_internal.h"

namespace {

using ssd::kChunk;
using ssd::kPGroup;

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// An integer from the environment (tuning overrides), or dflt.
int getenv_int(const char* name, int dflt) {
    const char* e = getenv(name);
    return e && e[0] ? atoi(e) : dflt;
}

struct Plan {
    int32_t K = 1;          // chunks per span
    int32_t sps = 0;        // spans per sequence (batch mode)
    int32_t npg = 0;        // headdim column groups
    int32_t hg_state = 1;   // heads per span_state workgroup
    int32_t hg_scan = 1;    // heads per span_scan workgroup
    int32_t fuse = 0;       // 1: span_scan forms incoming states (no state_pass
                            // launch); 2: one fused launch does every stage
    int32_t hw_npb = 0;     // head-wave kernels: 16-column blocks per wave;
                            // 0 = span kernels
    int64_t nspan = 0;      // span slots
    size_t off_sync = 0, off_states = 0, off_decay = 0, off_cu = 0, off_spoff = 0, off_table = 0;
    size_t total = 0;
};

// Chunks per span: the state stays on chip inside a span and only span
// borders go through HBM, so longer spans move fewer bytes; but each span is
// walked by one workgroup, so spans stay short enough that the span_scan grid
// keeps >= 4096 workgroups (16 per CU) once past four chunks.
// SSD_SPAN_CHUNKS overrides it (tuning sweeps).
int32_t choose_k(int64_t nch, int64_t groups) {
    if (const char* e = getenv("SSD_SPAN_CHUNKS")) {
        const int v = atoi(e);
        if (v >= 1 && v <= 64) return v;
    }
    // Four-chunk spans, or eight when that still leaves >= 1024 span x
    // head-group items (the wide workload: 8-chunk spans run 15 % faster)
    int32_t K = 4;
    while (K < 8 && ceil_div(nch, K) * groups >= 2048) K *= 2;
    return K;
}

// Head-wave kernels (bf16, d_state 64 / 128): a head's work for a chunk in
// one wave per 32 headdim columns (npb 2) or 64 (npb 4, d_state 64 only).
// Their per-chunk pipeline is cheaper than the span kernels' but needs long
// spans to pay for the state pass, so they serve problems with at least
// 16384 chunk-head-column-group work items (on one MI355X the span kernels
// are faster below that: 119 vs 146 us on 8192 tokens x 80 heads).  Spans: the longest of 32, 16, ... chunks that
// still give >= 2048 waves; 4 heads per workgroup at d_state 128 (they share
// the B / C tiles and the causal C B^T), 2 at d_state 64.
// SSD_KERNEL=span|hw forces a family; SSD_HW_NPB, SSD_HW_HEADS and
// SSD_SPAN_CHUNKS override the shape (tuning sweeps).
bool choose_hw(int64_t nch, int64_t heads, int64_t npg, int32_t hpg, int32_t N, int32_t* K,
               int32_t* npb, int32_t* hg) {
    const char* kf = getenv("SSD_KERNEL");
    if (kf && strcmp(kf, "span") == 0) return false;
    const bool forced = kf && strcmp(kf, "hw") == 0;
    if (!forced && nch * heads * npg < 16384) return false;
    int32_t b = 2;
    auto waves = [&](int32_t k) { return ceil_div(nch, k) * heads * npg * (4 / b); };
    int32_t k = 32;
    while (k > 1 && waves(k) < 2048) k /= 2;
    int32_t g = N >= 128 ? 4 : 2;
    while (hpg % g) g /= 2;
    if (const char* e = getenv("SSD_HW_NPB")) {
        const int v = atoi(e);
        if (v == 2 || (v == 4 && N <= 64)) b = v;
    }
    if (const char* e = getenv("SSD_HW_HEADS")) {
        const int v = atoi(e);
        if ((v == 1 || v == 2 || v == 4) && hpg % v == 0) g = v;
    }
    if (const char* e = getenv("SSD_SPAN_CHUNKS")) {
        const int v = atoi(e);
        if (v >= 1 && v <= 64) k = v;
    }
    *K = k;
    *npb = b;
    *hg = g;
    return true;
}

// Heads per workgroup: `dflt` unless the named environment variable asks
// for 1 or 2 up to `most` (tuning sweeps).  Both span kernels run one head
// per workgroup by default: more, smaller workgroups overlap their load,
// compute and store phases better than wider ones sharing B and C.
int32_t heads_override(const char* name, int32_t dflt, int32_t most) {
    if (const char* e = getenv(name)) {
        const int v = atoi(e);
        if ((v == 1 || v == 2) && v <= most) return v;
    }
    return dflt < most ? dflt : most;
}

int make_plan(const ssd_dims* d, Plan* pl) {
    if (!d) return SSD_ERR_NULL_ARG;
    if (d->dtype != SSD_F32 && d->dtype != SSD_BF16) return SSD_ERR_DTYPE;
    if (d->batch < 1 || d->seqlen < 0 || d->nheads < 1 || d->ngroups < 1 || d->nseq < 0)
        return SSD_ERR_SHAPE;
    if (d->nheads % d->ngroups != 0) return SSD_ERR_SHAPE;
    if (d->headdim < 16 || d->headdim % 16 != 0 || d->headdim > 512) return SSD_ERR_SHAPE;
    if (d->d_state < 1 || d->d_state > 4096) return SSD_ERR_SHAPE;
    if (d->chunk_size != kChunk) return SSD_ERR_UNSUPPORTED;
    if (ssd::span_lds_bytes(d->dtype, d->d_state, true) == 0) return SSD_ERR_UNSUPPORTED;
    if (d->nseq > 0 && d->batch != 1) return SSD_ERR_SHAPE;
    const int64_t T = (int64_t)d->batch * d->seqlen;
    if (d->nseq > 0 && T > INT32_MAX) return SSD_ERR_SHAPE;
    if (T > ((int64_t)1 << 40)) return SSD_ERR_SHAPE;

    pl->npg = (int32_t)ceil_div(d->headdim, kPGroup);
    // heads per workgroup: as many as the kernel carries, all in one B/C group
    const int32_t hpg = d->nheads / d->ngroups;
    pl->hg_state = heads_override("SSD_HEADS_STATE", 1, ssd::span_max_heads(d->dtype, d->d_state, false));
    while (hpg % pl->hg_state) pl->hg_state /= 2;
    pl->hg_scan = heads_override("SSD_HEADS_SCAN", 1, ssd::span_max_heads(d->dtype, d->d_state, true));
    while (hpg % pl->hg_scan) pl->hg_scan /= 2;
    const int64_t nch_bound = d->nseq > 0 ? ceil_div(T, kChunk) + d->nseq
                                          : (int64_t)d->batch * ceil_div(d->seqlen, kChunk);
    pl->K = choose_k(nch_bound, ceil_div(d->nheads, pl->hg_scan) * pl->npg);
    // Large bf16 problems with d_state 64 or 128 run the head-wave kernels.
    if (d->dtype == SSD_BF16 && (d->d_state == 64 || d->d_state == 128)) {
        int32_t K, npb, hg;
        if (choose_hw(nch_bound, d->nheads, pl->npg, hpg, d->d_state, &K, &npb, &hg) &&
            ssd::hw_supported(d->dtype, d->d_state, hg, npb)) {
            pl->K = K;
            pl->hw_npb = npb;
            // The state kernel groups at most two heads (four at d_state 128
            // made it slower: 76 vs 62 us on the packed workload); span
            // states are stored per head, so it need not match the scan.
            pl->hg_scan = hg;
            pl->hg_state = hg > 2 ? 2 : hg;
            if (const char* e = getenv("SSD_HW_HEADS_STATE")) {
                const int v = atoi(e);
                if ((v == 1 || v == 2 || v == 4) && hpg % v == 0 &&
                    ssd::hw_supported(d->dtype, d->d_state, v, npb))
                    pl->hg_state = v;
            }
        }
    }
    if (d->nseq > 0) {
        pl->sps = 0;
        pl->nspan = ceil_div(T, (int64_t)kChunk * pl->K) + d->nseq;
    } else {
        pl->sps = (int32_t)ceil_div(ceil_div(d->seqlen, kChunk), pl->K);
        pl->nspan = (int64_t)d->batch * pl->sps;
        // Few spans per sequence (up to 8): span_scan folds the earlier span
        // states of its sequence itself, which saves the state_pass launch
        // (with 16 the fold's re-reads cost more than the launch).  Empty
        // sequences keep the three launches (state_pass copies init_state to
        // final_state).  SSD_FUSE_PASS=0 / 1 / 2 forces the three launches,
        // these two, or one fused launch whose workgroups hand the span
        // states to the later spans of their sequence (as fast as the two
        // launches at the sizes measured, so not the default).
        const int64_t work = pl->nspan * ceil_div(d->nheads, pl->hg_scan) * pl->npg;
        pl->fuse = pl->sps > 0 && pl->sps <= 8 ? 1 : 0;
        if (const char* e = getenv("SSD_FUSE_PASS")) {
            if (e[0] >= '0' && e[0] <= '2' && e[1] == 0) pl->fuse = e[0] - '0';
        }
        if (pl->sps == 0 || pl->hw_npb) pl->fuse = 0;  // head-wave: three launches
        if (pl->fuse == 2 && work >= ((int64_t)1 << 31)) pl->fuse = 1;
    }
    // The span kernels decode their work items in 32 bits.
    if (pl->nspan * d->nheads * pl->npg >= ((int64_t)1 << 31)) return SSD_ERR_SHAPE;
    // The header sits at the start of every plan's workspace; the fused
    // launch's words follow it: one 64-bit ticket/epoch word per chain
    // (sequence, head group, column group), then one flag per workgroup.
    size_t off = 0;
    pl->off_sync = off;
    off = align_up(off + ssd::kSyncHeader * sizeof(uint32_t));
    if (pl->fuse == 2) {
        const int64_t chains = (int64_t)d->batch * ceil_div(d->nheads, pl->hg_scan) * pl->npg;
        off = align_up(off + (size_t)chains * sizeof(uint64_t) +
                       (size_t)pl->nspan * ceil_div(d->nheads, pl->hg_scan) * pl->npg * sizeof(uint32_t));
    }
    pl->off_states = off;
    const size_t esz = d->dtype == SSD_BF16 ? 2 : 4;  // span states use the input type
    off = align_up(off + (size_t)pl->nspan * d->nheads * d->headdim * d->d_state * esz);
    pl->off_decay = off;
    off = align_up(off + (size_t)pl->nspan * d->nheads * sizeof(float));
    if (d->nseq > 0) {
        pl->off_cu = off;
        off = align_up(off + (size_t)(d->nseq + 1) * sizeof(int32_t));
        pl->off_spoff = off;
        off = align_up(off + (size_t)(d->nseq + 1) * sizeof(int32_t));
        pl->off_table = off;
        off = align_up(off + (size_t)pl->nspan * sizeof(int4));
    }
    pl->total = off;
    return SSD_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Backward plan.  Every chunk is its own span, so the two state passes
// leave the state entering every chunk (forward direction) and the gradient
// of the state leaving every chunk (walking the chunks backwards) in the
// workspace; the gradient kernel then treats the chunks independently.  Its
// workgroups take hs heads of one B/C group; hs is the largest divisor of
// the group's heads that still gives >= 256 workgroups, one per CU (the
// kernel's LDS allows one; SSD_BWD_HEADS overrides it), and the head
// subsets' dB / dC partials are added after it.
struct BPlan {
    int64_t nchunk = 0;    // chunk slots
    int32_t cps = 0;       // chunks per sequence (batch mode)
    int32_t nsub = 1, hs = 1;
    size_t off_cu = 0, off_spoff = 0, off_table = 0;
    int64_t nspan4 = 0;    // (varlen) four-chunk span slots of the chunk-state pass
    size_t off_cu4 = 0, off_spoff4 = 0, off_table4 = 0;
    size_t off_sa = 0, off_da = 0, off_sb = 0, off_db = 0;
    size_t off_pb = 0, off_pc = 0, off_pi = 0, total = 0;
};

int make_bwd_plan(const ssd_dims* d, BPlan* bp) {
    Plan pl;
    const int st = make_plan(d, &pl);  // the forward's size checks
    if (st != SSD_OK) return st;
    if (!ssd::bwd_supported(d->dtype, d->d_state)) return SSD_ERR_UNSUPPORTED;
    const int64_t T = (int64_t)d->batch * d->seqlen;
    bp->cps = (int32_t)ceil_div(d->seqlen, kChunk);
    bp->nchunk = d->nseq > 0 ? ceil_div(T, kChunk) + d->nseq : (int64_t)d->batch * bp->cps;
    const int32_t hpg = d->nheads / d->ngroups;
    int32_t hs = 1;
    for (int32_t v = hpg; v >= 1; --v) {
        if (hpg % v == 0 && v <= ssd::kBwdMaxHeads && bp->nchunk * d->ngroups * (hpg / v) >= 256) {
            hs = v;
            break;
        }
    }
    if (const char* e = getenv("SSD_BWD_HEADS")) {
        const int v = atoi(e);
        if (v >= 1 && v <= hpg && v <= ssd::kBwdMaxHeads && hpg % v == 0) hs = v;
    }
    bp->hs = hs;
    bp->nsub = hpg / hs;
    const size_t esz = d->dtype == SSD_BF16 ? 2 : 4;
    const size_t states = (size_t)bp->nchunk * d->nheads * d->headdim * d->d_state * esz;
    const size_t part = (size_t)bp->nsub * T * d->ngroups * d->d_state * sizeof(float);
    size_t off = align_up(ssd::kSyncHeader * sizeof(uint32_t));
    if (d->nseq > 0) {
        bp->off_cu = off;
        off = align_up(off + (size_t)(d->nseq + 1) * sizeof(int32_t));
        bp->off_spoff = off;
        off = align_up(off + (size_t)(d->nseq + 1) * sizeof(int32_t));
        bp->off_table = off;
        off = align_up(off + (size_t)bp->nchunk * sizeof(int4));
        bp->nspan4 = ceil_div(T, (int64_t)kChunk * 4) + d->nseq;
        bp->off_cu4 = off;
        off = align_up(off + (size_t)(d->nseq + 1) * sizeof(int32_t));
        bp->off_spoff4 = off;
        off = align_up(off + (size_t)(d->nseq + 1) * sizeof(int32_t));
        bp->off_table4 = off;
        off = align_up(off + (size_t)bp->nspan4 * sizeof(int4));
    }
    bp->off_sa = off;
    off = align_up(off + states);
    bp->off_da = off;
    off = align_up(off + (size_t)bp->nchunk * d->nheads * sizeof(float));
    bp->off_sb = off;
    off = align_up(off + states);
    bp->off_db = off;
    off = align_up(off + (size_t)bp->nchunk * d->nheads * sizeof(float));
    bp->off_pb = off;
    off = align_up(off + part);
    bp->off_pc = off;
    off = align_up(off + part);
    bp->off_pi = off;
    off = align_up(off + (size_t)bp->nchunk * d->ngroups * bp->nsub * sizeof(float));
    bp->total = off;
    return SSD_OK;
}

// SSD_CHECK=1: copy cu_seqlens to the host (synchronizes the stream) and
// check 0 = cu[0] <= cu[1] <= ... <= cu[nseq] = L.
int check_cu(const int32_t* cu, int32_t nseq, int64_t T, hipStream_t s) {
    std::vector<int32_t> h(nseq + 1);
    if (hipMemcpyAsync(h.data(), cu, sizeof(int32_t) * (nseq + 1), hipMemcpyDeviceToHost, s) !=
        hipSuccess)
        return SSD_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return SSD_ERR_HIP;
    if (h[0] != 0 || h[nseq] != T) return SSD_ERR_CU_SEQLENS;
    for (int32_t i = 0; i < nseq; ++i)
        if (h[i + 1] < h[i]) return SSD_ERR_CU_SEQLENS;
    return SSD_OK;
}

}  // namespace

extern "C" {

int ssd_abi_version(void) { return SSD_ABI_VERSION; }

size_t ssd_fwd_workspace_bytes(const ssd_dims* dims) {
    Plan pl;
    if (make_plan(dims, &pl) != SSD_OK) return 0;
    return pl.total;
}

const char* ssd_status_string(int status) {
    switch (status) {
        case SSD_OK: return "SSD_OK: success";
        case SSD_ERR_NULL_ARG: return "SSD_ERR_NULL_ARG: a required pointer is NULL";
        case SSD_ERR_SHAPE: return "SSD_ERR_SHAPE: inconsistent or out-of-range sizes or strides";
        case SSD_ERR_DTYPE: return "SSD_ERR_DTYPE: unknown dtype code";
        case SSD_ERR_ALIGN: return "SSD_ERR_ALIGN: pointer or stride not 16-byte aligned";
        case SSD_ERR_UNSUPPORTED:
            return "SSD_ERR_UNSUPPORTED: chunk_size or d_state not built into this library";
        case SSD_ERR_WORKSPACE: return "SSD_ERR_WORKSPACE: workspace missing or too small";
        case SSD_ERR_HIP: return "SSD_ERR_HIP: a HIP runtime call or kernel launch failed";
        case SSD_ERR_CU_SEQLENS:
            return "SSD_ERR_CU_SEQLENS: cu_seqlens not 0..L and non-decreasing";
    }
    return "unknown ssd status";
}

int ssd_fwd_plan(const ssd_dims* dims, ssd_plan_info* out) {
    Plan pl;
    const int st = make_plan(dims, &pl);
    if (st != SSD_OK) return st;
    if (!out) return SSD_ERR_NULL_ARG;
    out->chunks_per_span = pl.K;
    out->col_groups = pl.npg;
    out->nspan = pl.nspan;
    out->workspace_bytes = pl.total;
    out->fused_pass = pl.fuse;
    out->heads_per_wg = pl.hg_scan;
    out->cols_per_wave = pl.hw_npb ? 16 * pl.hw_npb : 16;
    out->head_wave = pl.hw_npb ? 1 : 0;
    return SSD_OK;
}

int ssd_fwd(const ssd_dims* dims, const void* x, const void* d_raw, float d_init, const void* B,
            const void* C, const float* init_state, const int32_t* cu_seqlens, int32_t reverse,
            void* y, int64_t y_token_stride, int64_t y_head_stride, float* final_state,
            void* workspace, size_t workspace_bytes, void* stream) {
    return ssd_fwd_stages(SSD_STAGE_ALL, dims, x, d_raw, d_init, B, C, init_state, cu_seqlens,
                          reverse, y, y_token_stride, y_head_stride, final_state, workspace,
                          workspace_bytes, stream);
}

int ssd_fwd_stages(uint32_t mask, const ssd_dims* dims, const void* x, const void* d_raw,
                   float d_init, const void* B, const void* C, const float* init_state,
                   const int32_t* cu_seqlens, int32_t reverse, void* y, int64_t y_token_stride,
                   int64_t y_head_stride, float* final_state, void* workspace,
                   size_t workspace_bytes, void* stream) {
    if (mask & ~(uint32_t)SSD_STAGE_ALL) return SSD_ERR_SHAPE;
    Plan pl;
    const int st = make_plan(dims, &pl);
    if (st != SSD_OK) return st;
    const ssd_dims& d = *dims;
    const int64_t T = (int64_t)d.batch * d.seqlen;
    if (T > 0 && (!x || !d_raw || !B || !C || !y)) return SSD_ERR_NULL_ARG;
    if (d.nseq > 0 && !cu_seqlens) return SSD_ERR_NULL_ARG;
    if (d.nseq == 0 && cu_seqlens) return SSD_ERR_SHAPE;
    if (reverse != 0 && reverse != 1) return SSD_ERR_SHAPE;
    const int64_t esz = d.dtype == SSD_BF16 ? 2 : 4;
    const int64_t per_unit = 16 / esz;
    if (!aligned16(x) || !aligned16(B) || !aligned16(C) || !aligned16(y)) return SSD_ERR_ALIGN;
    if ((uintptr_t)d_raw % esz) return SSD_ERR_ALIGN;  // read one element per lane
    if (y_token_stride % per_unit != 0 || y_head_stride % per_unit != 0) return SSD_ERR_ALIGN;
    if (y_token_stride < 0 || y_head_stride < 0) return SSD_ERR_SHAPE;
    if (y_token_stride > ((int64_t)1 << 24)) return SSD_ERR_SHAPE;
    if (((uintptr_t)init_state & 3u) || ((uintptr_t)final_state & 3u)) return SSD_ERR_ALIGN;
    if (pl.total > 0) {
        if (!workspace || workspace_bytes < pl.total) return SSD_ERR_WORKSPACE;
        if ((uintptr_t)workspace % kAlign) return SSD_ERR_ALIGN;
    }
    hipStream_t s = (hipStream_t)stream;
    if (d.nseq > 0 && (mask & SSD_STAGE_TABLE)) {
        const char* chk = getenv("SSD_CHECK");
        if (chk && chk[0] == '1') {
            const int c = check_cu(cu_seqlens, d.nseq, T, s);
            if (c != SSD_OK) return c;
        }
    }

    char* ws = (char*)workspace;
    ssd::KParams p;
    memset(&p, 0, sizeof(p));
    p.x = x;
    p.d_raw = d_raw;
    p.B = B;
    p.C = C;
    p.y = y;
    p.init = init_state;
    p.final_state = final_state;
    p.states = ws + pl.off_states;
    p.decay = (float*)(ws + pl.off_decay);
    p.L = d.seqlen;
    p.ys_t = y_token_stride;
    p.ys_h = y_head_stride;
    p.xs_t = (int64_t)d.nheads * d.headdim;
    p.xs_h = d.headdim;
    p.nspan = pl.nspan;
    p.batch = d.batch;
    p.H = d.nheads;
    p.P = d.headdim;
    p.G = d.ngroups;
    p.N = d.d_state;
    p.nseq = d.nseq;
    p.K = pl.K;
    p.sps = pl.sps;
    p.npg = pl.npg;
    p.hg_state = pl.hg_state;
    p.hg_scan = pl.hg_scan;
    p.reverse = reverse;
    p.fuse_pass = pl.fuse;
    p.hw_npb = pl.hw_npb;
    p.sync = (uint32_t*)(ws + pl.off_sync);
    p.d_init = d_init;

    hipError_t e = hipSuccess;
    if (d.nseq > 0) {
        p.cu = (const int32_t*)(ws + pl.off_cu);
        p.span_off = (const int32_t*)(ws + pl.off_spoff);
        p.table = (const int4*)(ws + pl.off_table);
        if (mask & SSD_STAGE_TABLE) {
            e = ssd::launch_span_table(cu_seqlens, d.nseq, T, pl.K, pl.nspan,
                                       (int32_t*)(ws + pl.off_cu), (int32_t*)(ws + pl.off_spoff),
                                       (int4*)(ws + pl.off_table), s);
            if (e != hipSuccess) return SSD_ERR_HIP;
        }
    }
    if ((mask & SSD_STAGE_STATE) && pl.fuse != 2) {
        e = pl.hw_npb ? ssd::launch_hw_state(p, d.d_state, s)
                      : ssd::launch_span_state(p, d.dtype, d.d_state, s);
        if (e != hipSuccess) return SSD_ERR_HIP;
    }
    if ((mask & SSD_STAGE_PASS) && !pl.fuse) {
        e = ssd::launch_state_pass(p, d.dtype, s);
        if (e != hipSuccess) return SSD_ERR_HIP;
    }
    if (mask & SSD_STAGE_SCAN) {
        e = pl.hw_npb ? ssd::launch_hw_scan(p, d.d_state, s)
                      : ssd::launch_span_scan(p, d.dtype, d.d_state, s);
        if (e != hipSuccess) return SSD_ERR_HIP;
    }
    return SSD_OK;
}

size_t ssd_bwd_workspace_bytes(const ssd_dims* dims) {
    BPlan bp;
    if (make_bwd_plan(dims, &bp) != SSD_OK) return 0;
    return bp.total;
}

int ssd_bwd(const ssd_dims* dims, const void* x, const void* d_raw, float d_init, const void* B,
            const void* C, const float* init_state, const int32_t* cu_seqlens, int32_t reverse,
            const void* y, int64_t y_token_stride, int64_t y_head_stride, const void* dy,
            int64_t dy_token_stride, int64_t dy_head_stride, const float* d_final, void* dx,
            void* dd_raw, void* dB, void* dC, float* dinit_state, float* dd_init, void* workspace,
            size_t workspace_bytes, void* stream) {
    BPlan bp;
    const int st = make_bwd_plan(dims, &bp);
    if (st != SSD_OK) return st;
    const ssd_dims& d = *dims;
    const int64_t T = (int64_t)d.batch * d.seqlen;
    if (T > 0 && (!x || !d_raw || !B || !C || !y || !dy || !dx || !dd_raw || !dB || !dC))
        return SSD_ERR_NULL_ARG;
    if (d.nseq > 0 && !cu_seqlens) return SSD_ERR_NULL_ARG;
    if (d.nseq == 0 && cu_seqlens) return SSD_ERR_SHAPE;
    if (reverse != 0 && reverse != 1) return SSD_ERR_SHAPE;
    const int64_t esz = d.dtype == SSD_BF16 ? 2 : 4;
    const int64_t per_unit = 16 / esz;
    if (!aligned16(x) || !aligned16(B) || !aligned16(C) || !aligned16(y) || !aligned16(dy) ||
        !aligned16(dx) || !aligned16(dB) || !aligned16(dC))
        return SSD_ERR_ALIGN;
    if (((uintptr_t)d_raw % esz) || ((uintptr_t)dd_raw % esz)) return SSD_ERR_ALIGN;
    for (int64_t v : {y_token_stride, y_head_stride, dy_token_stride, dy_head_stride}) {
        if (v % per_unit != 0) return SSD_ERR_ALIGN;
        if (v < 0 || v > ((int64_t)1 << 24)) return SSD_ERR_SHAPE;
    }
    if (((uintptr_t)init_state & 3u) || ((uintptr_t)d_final & 3u) || ((uintptr_t)dinit_state & 3u) ||
        ((uintptr_t)dd_init & 3u))
        return SSD_ERR_ALIGN;
    if (!workspace || workspace_bytes < bp.total) return SSD_ERR_WORKSPACE;
    if ((uintptr_t)workspace % kAlign) return SSD_ERR_ALIGN;
    hipStream_t s = (hipStream_t)stream;
    if (d.nseq > 0) {
        const char* chk = getenv("SSD_CHECK");
        if (chk && chk[0] == '1') {
            const int c = check_cu(cu_seqlens, d.nseq, T, s);
            if (c != SSD_OK) return c;
        }
    }
    char* ws = (char*)workspace;
    hipError_t e = hipSuccess;

    // state entering every chunk: the forward's span kernels, one chunk per span
    ssd::KParams pa;
    memset(&pa, 0, sizeof(pa));
    pa.x = x;
    pa.d_raw = d_raw;
    pa.B = B;
    pa.C = C;
    pa.init = init_state;
    pa.states = ws + bp.off_sa;
    pa.decay = (float*)(ws + bp.off_da);
    pa.L = d.seqlen;
    pa.xs_t = (int64_t)d.nheads * d.headdim;
    pa.xs_h = d.headdim;
    pa.nspan = bp.nchunk;
    pa.batch = d.batch;
    pa.H = d.nheads;
    pa.P = d.headdim;
    pa.G = d.ngroups;
    pa.N = d.d_state;
    pa.nseq = d.nseq;
    pa.K = 1;
    pa.sps = d.nseq > 0 ? 0 : bp.cps;
    pa.npg = (int32_t)ceil_div(d.headdim, kPGroup);
    pa.hg_state = pa.hg_scan = 1;
    pa.reverse = reverse;
    pa.sync = (uint32_t*)ws;
    pa.d_init = d_init;
    if (d.nseq > 0) {
        pa.cu = (const int32_t*)(ws + bp.off_cu);
        pa.span_off = (const int32_t*)(ws + bp.off_spoff);
        pa.table = (const int4*)(ws + bp.off_table);
        e = ssd::launch_span_table(cu_seqlens, d.nseq, T, 1, bp.nchunk, (int32_t*)(ws + bp.off_cu),
                                   (int32_t*)(ws + bp.off_spoff), (int4*)(ws + bp.off_table), s);
        if (e != hipSuccess) return SSD_ERR_HIP;
    }

    // gradient of the state leaving every chunk: the same kernels on (C, dy)
    // with weights e^{cs_s}, walked from the last chunk back from d_final;
    // what is left after the first chunk is the initial state's gradient.
    // The two directions are independent: each kernel pair is one launch.
    ssd::KParams pg = pa;
    pg.x = dy;
    pg.xs_t = dy_token_stride;
    pg.xs_h = dy_head_stride;
    pg.B = C;
    pg.init = d_final;
    pg.final_state = dinit_state;
    pg.states = ws + bp.off_sb;
    pg.decay = (float*)(ws + bp.off_db);
    pg.wmode = 1;
    pg.pass_desc = 1;
    // Each chunk-state workgroup walks up to four chunks of a sequence (its
    // loads double-buffered) and stores every chunk's local state: the same
    // states as one workgroup per chunk, with a quarter of the workgroup
    // set-up.  With cu_seqlens the walks follow a second span table of
    // four-chunk spans, and the chunk slots are the per-chunk table's.
    ssd::KParams pa4 = pa, pg4 = pg;
    if (getenv_int("SSD_BWD_STATE_CHUNKS", 4) == 4) {
        if (d.nseq > 0) {
            e = ssd::launch_span_table(cu_seqlens, d.nseq, T, 4, bp.nspan4,
                                       (int32_t*)(ws + bp.off_cu4), (int32_t*)(ws + bp.off_spoff4),
                                       (int4*)(ws + bp.off_table4), s);
            if (e != hipSuccess) return SSD_ERR_HIP;
        }
        for (ssd::KParams* k : {&pa4, &pg4}) {
            k->K = 4;
            k->chunk_out = 1;
            if (d.nseq > 0) {
                k->nspan = bp.nspan4;
                k->cu = (const int32_t*)(ws + bp.off_cu4);
                k->span_off = (const int32_t*)(ws + bp.off_spoff4);
                k->table = (const int4*)(ws + bp.off_table4);
                k->chunk_slot = (const int32_t*)(ws + bp.off_spoff);
            } else {
                k->sps = (int32_t)ceil_div(bp.cps, 4);
                k->nspan = (int64_t)d.batch * k->sps;
            }
        }
    }
    e = ssd::launch_span_state_pair(pa4, pg4, d.dtype, d.d_state, s);
    if (e == hipSuccess) e = ssd::launch_state_pass_pair(pa, pg, d.dtype, s);
    if (e != hipSuccess) return SSD_ERR_HIP;

    ssd::BParams q;
    memset(&q, 0, sizeof(q));
    q.x = x;
    q.d_raw = d_raw;
    q.B = B;
    q.C = C;
    q.y = y;
    q.dy = dy;
    q.hprev = ws + bp.off_sa;
    q.gout = ws + bp.off_sb;
    q.dx = dx;
    q.dd_raw = dd_raw;
    q.dB_part = (float*)(ws + bp.off_pb);
    q.dC_part = (float*)(ws + bp.off_pc);
    q.ddi_part = (float*)(ws + bp.off_pi);
    q.cu = pa.cu;
    q.table = pa.table;
    q.L = d.seqlen;
    q.ntok = T;
    q.xs_t = (int64_t)d.nheads * d.headdim;
    q.xs_h = d.headdim;
    q.ys_t = y_token_stride;
    q.ys_h = y_head_stride;
    q.gs_t = dy_token_stride;
    q.gs_h = dy_head_stride;
    q.nchunk = bp.nchunk;
    q.batch = d.batch;
    q.H = d.nheads;
    q.P = d.headdim;
    q.G = d.ngroups;
    q.N = d.d_state;
    q.nseq = d.nseq;
    q.cps = bp.cps;
    q.nsub = bp.nsub;
    q.hs = bp.hs;
    q.reverse = reverse;
    q.d_init = d_init;
    e = ssd::launch_bwd_chunk(q, d.dtype, s);
    if (e == hipSuccess) e = ssd::launch_bwd_reduce(q, d.dtype, dB, dC, dd_init, s);
    return e == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

}  // extern "C"
