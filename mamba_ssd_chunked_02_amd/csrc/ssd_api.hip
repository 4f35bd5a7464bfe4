// C ABI of libssd: argument checks, planning and the launch sequence.
// Every check runs on the host before anything is launched.
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "../../include/ssd.h"
#include "ssd_internal.h"

namespace {

using ssd::kChunk;
using ssd::kPGroup;

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

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
    int32_t state_f32 = 0;  // span states stored in float32
    int64_t nspan = 0;      // span slots
    int64_t nsync = 0;      // 32-bit words the fused launch resets (plan 2)
    size_t off_sync = 0, off_states = 0, off_decay = 0, off_cu = 0, off_spoff = 0, off_table = 0;
    size_t total = 0;
};

const ssd_tuning kNoTuning = {};

// Chunks per span: the state stays on chip inside a span and only span
// borders go through HBM, so longer spans move fewer bytes; but each span is
// walked by one workgroup, so spans stay short enough to keep the grid wide.
// Four-chunk spans, or eight when that still leaves >= 2048 span x
// head-group items (8192 tokens x 80 heads: 8-chunk spans run 15 % faster).
// A grid narrower than the chip's 256 CUs takes shorter spans (fewer chunk
// steps in a row, more workgroups), down to one chunk, as long as a sequence
// keeps at most eight spans so the scan still folds them itself (256 tokens
// x 2 heads: 11.3 us with one-chunk spans, 22.4 with four).  cps: chunks per
// sequence, 0 for packed sequences.
int32_t choose_k(int64_t nch, int64_t groups, int64_t cps) {
    int32_t K = 4;
    while (K < 8 && ceil_div(nch, K) * groups >= 2048) K *= 2;
    while (K > 1 && cps > 0 && ceil_div(nch, K) * groups < 256 && ceil_div(cps, K / 2) <= 8) K /= 2;
    return K;
}

// Head-wave kernels (bf16, d_state 64 / 128): a head's work for a chunk in
// one wave per 32 headdim columns (npb 2) or 64 (npb 4, d_state 64 only).
// Their per-chunk pipeline is cheaper than the span kernels' but needs long
// spans to pay for the state pass, so the planner takes them for problems
// with at least 16384 chunk-head-column-group work items (on one MI355X the
// span kernels are faster below that: 119 vs 146 us on 8192 tokens x 80
// heads).  Spans: 64 chunks where that still gives >= 8192 waves (1M tokens
// x 8 heads x 192: 4.62 vs 4.73 ms per bidirectional step with 32), else the
// longest of 32, 16, ... chunks that still give >= 2048 waves; 4 heads per
// workgroup at d_state 128 (they share the B / C tiles and the causal
// C B^T), 2 at d_state 64.
bool choose_hw(const ssd_tuning& t, int64_t nch, int64_t heads, int64_t npg, int32_t hpg,
               int32_t N, int32_t* K, int32_t* npb, int32_t* hg) {
    if (t.kernel == 1) return false;
    if (t.kernel != 2 && nch * heads * npg < 16384) return false;
    int32_t b = t.cols_per_wave ? t.cols_per_wave / 16 : 2;
    auto waves = [&](int32_t k) { return ceil_div(nch, k) * heads * npg * (4 / b); };
    int32_t k = waves(64) >= 8192 ? 64 : 32;
    while (k > 1 && waves(k) < 2048) k /= 2;
    int32_t g = N >= 128 ? 4 : 2;
    while (hpg % g) g /= 2;
    if (t.heads_scan) g = t.heads_scan;
    *K = t.chunks_per_span ? t.chunks_per_span : k;
    *npb = b;
    *hg = g;
    return true;
}

int make_plan(const ssd_dims* d, const ssd_tuning* tun, Plan* pl) {
    if (!d) return SSD_ERR_NULL_ARG;
    const ssd_tuning& t = tun ? *tun : kNoTuning;
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
    // tuning values in range
    for (int32_t r : t.reserved)
        if (r) return SSD_ERR_SHAPE;
    if (t.kernel < 0 || t.kernel > 2 || t.chunks_per_span < 0 || t.chunks_per_span > 64 ||
        t.state_pass < 0 || t.state_pass > 3 || t.heads_state < 0 || t.heads_scan < 0 ||
        (t.cols_per_wave != 0 && t.cols_per_wave != 32 && t.cols_per_wave != 64) ||
        t.bwd_heads < 0 || (t.bwd_state_chunks != 0 && t.bwd_state_chunks != 1 &&
                            t.bwd_state_chunks != 4) ||
        t.state_f32 < 0 || t.state_f32 > 1)
        return SSD_ERR_SHAPE;
    const int32_t hpg = d->nheads / d->ngroups;
    if (t.bwd_heads && (hpg % t.bwd_heads || t.bwd_heads > ssd::kBwdMaxHeads)) return SSD_ERR_SHAPE;
    const bool hw_ok = d->dtype == SSD_BF16 && (d->d_state == 64 || d->d_state == 128);
    if (t.kernel == 2 && !hw_ok) return SSD_ERR_UNSUPPORTED;
    if (t.kernel == 2 && t.state_f32) return SSD_ERR_SHAPE;
    if (t.cols_per_wave == 64 && !(hw_ok && d->d_state == 64)) return SSD_ERR_SHAPE;

    pl->npg = (int32_t)ceil_div(d->headdim, kPGroup);
    pl->state_f32 = t.state_f32;
    // Span kernels carry one head per workgroup by default: more, smaller
    // workgroups overlap their load, compute and store phases better than
    // wider ones sharing B and C.
    const int32_t hs_max = ssd::span_max_heads(d->dtype, d->d_state, false);
    const int32_t hc_max = ssd::span_max_heads(d->dtype, d->d_state, true);
    pl->hg_state = t.heads_state ? t.heads_state : 1;
    pl->hg_scan = t.heads_scan ? t.heads_scan : 1;
    const int64_t nch_bound = d->nseq > 0 ? ceil_div(T, kChunk) + d->nseq
                                          : (int64_t)d->batch * ceil_div(d->seqlen, kChunk);
    pl->K = t.chunks_per_span ? t.chunks_per_span
                              : choose_k(nch_bound, ceil_div(d->nheads, pl->hg_scan) * pl->npg,
                                         d->nseq > 0 ? 0 : ceil_div(d->seqlen, kChunk));
    // Large bf16 problems with d_state 64 or 128 run the head-wave kernels.
    bool hw = false;
    if (hw_ok && !t.state_f32) {
        int32_t K, npb, hg;
        if (choose_hw(t, nch_bound, d->nheads, pl->npg, hpg, d->d_state, &K, &npb, &hg)) {
            // The state kernel groups at most two heads (four at d_state 128
            // made it slower: 76 vs 62 us on the packed workload); span
            // states are stored per head, so it need not match the scan.
            const int32_t hs = t.heads_state ? t.heads_state : (hg > 2 ? 2 : hg);
            hw = ssd::hw_supported(d->dtype, d->d_state, hg, npb) && hpg % hg == 0 &&
                 ssd::hw_supported(d->dtype, d->d_state, hs, npb) && hpg % hs == 0;
            // a shape asked for explicitly must exist; the planner's own
            // choice falls back to the span kernels
            if (!hw && (t.kernel == 2 || t.cols_per_wave)) return SSD_ERR_SHAPE;
            if (hw) {
                pl->K = K;
                pl->hw_npb = npb;
                pl->hg_scan = hg;
                pl->hg_state = hs;
            }
        }
    }
    if (!hw) {
        if (pl->hg_state > hs_max || pl->hg_scan > hc_max || pl->hg_state > 2 || pl->hg_scan > 2 ||
            hpg % pl->hg_state || hpg % pl->hg_scan)
            return SSD_ERR_SHAPE;
        if (t.cols_per_wave) return SSD_ERR_SHAPE;
    }
    if (d->nseq > 0) {
        pl->sps = 0;
        pl->nspan = ceil_div(T, (int64_t)kChunk * pl->K) + d->nseq;
        if (t.state_pass) return SSD_ERR_SHAPE;  // packed batches always take plan 0
    } else {
        pl->sps = (int32_t)ceil_div(ceil_div(d->seqlen, kChunk), pl->K);
        pl->nspan = (int64_t)d->batch * pl->sps;
        // Few spans per sequence (up to 8): span_scan folds the earlier span
        // states of its sequence itself, which saves the state_pass launch
        // (with 16 the fold's re-reads cost more than the launch).  Empty
        // sequences keep the three launches (state_pass copies init_state to
        // final_state).  Plan 2, one fused launch whose workgroups hand the
        // span states to the later spans of their sequence, is as fast as
        // plan 1 at the sizes measured, so only taken when asked for.
        pl->fuse = pl->sps > 0 && pl->sps <= 8 ? 1 : 0;
        if (t.state_pass) {
            if (hw && t.state_pass != 1) return SSD_ERR_SHAPE;  // head-wave: three launches
            if (pl->sps == 0 && t.state_pass != 1) return SSD_ERR_SHAPE;
            pl->fuse = t.state_pass - 1;
        }
        if (hw) pl->fuse = 0;
        if (pl->state_f32 && pl->fuse == 2) return SSD_ERR_SHAPE;
        const int64_t work = pl->nspan * ceil_div(d->nheads, pl->hg_scan) * pl->npg;
        if (pl->fuse == 2 && work >= ((int64_t)1 << 31)) return SSD_ERR_SHAPE;
    }
    // Span kernels: two heads per state workgroup (they share its B tile)
    // where that still leaves at least 128 state workgroups; with fewer,
    // one-head walks finish sooner (2 x 2048 tokens x 24 heads: 26.3 vs 26.6
    // us per step; 8192 tokens x 80 heads: 112.6 vs 113.7; 256 tokens x 2
    // heads: 11.0 vs 10.5).
    if (!hw && !t.heads_state && hpg % 2 == 0 && hs_max >= 2 &&
        pl->nspan * ceil_div(d->nheads, 2) * pl->npg >= 128)
        pl->hg_state = 2;
    // The span kernels decode their work items in 32 bits, and the state
    // pass its threads (four or eight state entries each).
    if (pl->nspan * d->nheads * pl->npg >= ((int64_t)1 << 31)) return SSD_ERR_SHAPE;
    const int64_t nstates = d->nseq > 0 ? d->nseq : d->batch;
    if (nstates * d->nheads * (int64_t)d->headdim * d->d_state >= ((int64_t)1 << 33))
        return SSD_ERR_SHAPE;
    // The header sits at the start of every plan's workspace; the fused
    // launch's words follow it: one 64-bit ticket/epoch word per chain
    // (sequence, head group, column group), then one flag per workgroup.
    size_t off = 0;
    pl->off_sync = off;
    off = align_up(off + ssd::kSyncHeader * sizeof(uint32_t));
    if (pl->fuse == 2) {
        const int64_t chains = (int64_t)d->batch * ceil_div(d->nheads, pl->hg_scan) * pl->npg;
        const int64_t words = 2 * chains + pl->nspan * ceil_div(d->nheads, pl->hg_scan) * pl->npg;
        pl->nsync = ssd::kSyncHeader + words;
        off = align_up(off + (size_t)words * sizeof(uint32_t));
    }
    pl->off_states = off;
    // span states: the input type, or float32 when asked for
    const size_t esz = (d->dtype == SSD_BF16 && !pl->state_f32) ? 2 : 4;
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

// Strides of every per-token tensor (elements): the caller's layout, or the
// contiguous one.
ssd_layout resolve_layout(const ssd_dims& d, const ssd_layout* lay) {
    if (lay) return *lay;
    ssd_layout l;
    l.x_token = l.y_token = l.dy_token = (int64_t)d.nheads * d.headdim;
    l.x_head = l.y_head = l.dy_head = d.headdim;
    l.d_raw_token = d.nheads;
    l.d_raw_head = 1;
    l.B_token = l.C_token = (int64_t)d.ngroups * d.d_state;
    l.B_group = l.C_group = d.d_state;
    return l;
}

// Stride rules: >= 0 and <= 2^24 elements; the 16-byte-row tensors' strides
// a multiple of 16 bytes.  The forward checks y's strides, the backward
// dy's (it does not read y).
int check_layout(const ssd_dims& d, const ssd_layout& l, bool bwd) {
    const int64_t esz = d.dtype == SSD_BF16 ? 2 : 4;
    const int64_t per_unit = 16 / esz;
    const int64_t lim = (int64_t)1 << 24;
    const int64_t out_t = bwd ? l.dy_token : l.y_token, out_h = bwd ? l.dy_head : l.y_head;
    const int64_t all[] = {l.x_token, l.x_head, l.d_raw_token, l.d_raw_head, l.B_token,
                           l.B_group, l.C_token, l.C_group, out_t, out_h};
    for (int64_t v : all)
        if (v < 0 || v > lim) return SSD_ERR_SHAPE;
    const int64_t rows[] = {l.x_token, l.x_head, l.B_token, l.B_group, l.C_token, l.C_group,
                            out_t, out_h};
    for (int64_t v : rows)
        if (v % per_unit) return SSD_ERR_ALIGN;
    return SSD_OK;
}

// Two [S, H, N, P] float32 state buffers: 0 when disjoint (or either is
// NULL), 1 when they are the same buffer, -1 when they partly overlap.
int state_alias(const void* a, const void* b, size_t bytes) {
    if (!a || !b || bytes == 0) return 0;
    if (a == b) return 1;
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return (x < y + bytes && y < x + bytes) ? -1 : 0;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Backward plan.  Every chunk is its own span, so the two state passes
// leave the state entering every chunk (forward direction) and the gradient
// of the state leaving every chunk (walking the chunks backwards) in the
// workspace; the gradient kernel then treats the chunks independently.  Its
// workgroups take hs heads of one B/C group; hs is the largest divisor of
// the group's heads that still gives >= 256 workgroups, one per CU (the
// kernel's LDS allows one; ssd_tuning.bwd_heads overrides it), and the
// head subsets' dB / dC partials are added after it.
struct BPlan {
    int64_t nchunk = 0;    // chunk slots
    int32_t cps = 0;       // chunks per sequence (batch mode)
    int32_t nsub = 1, hs = 1;
    size_t off_cu = 0, off_spoff = 0, off_table = 0;
    int32_t state_chunks = 4;  // chunks walked by one chunk-state workgroup
    int64_t nspan4 = 0;    // (varlen) four-chunk span slots of the chunk-state pass
    size_t off_cu4 = 0, off_spoff4 = 0, off_table4 = 0;
    size_t off_sa = 0, off_da = 0, off_sb = 0, off_db = 0;
    // (four-chunk walks) span-level states and decays of both sets
    int64_t nspan4s = 0;   // four-chunk span slots (batch or varlen)
    size_t off_ta = 0, off_ea = 0, off_tb = 0, off_eb = 0;
    size_t off_pb = 0, off_pc = 0, off_pi = 0, total = 0;
};

int make_bwd_plan(const ssd_dims* d, const ssd_tuning* tun, BPlan* bp) {
    Plan pl;
    const int st = make_plan(d, tun, &pl);  // the forward's size and tuning checks
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
    if (tun && tun->bwd_heads) hs = tun->bwd_heads;  // checked by make_plan
    // Four-chunk chunk-state walks, unless they leave fewer walks than the
    // chip has CUs (256 tokens x 2 heads: 24.0 us with one chunk per
    // workgroup, 27.0 with four; the layer workload: 85.6 vs 93.8).
    {
        const int64_t walks = (d->nseq > 0 ? ceil_div(T, (int64_t)kChunk * 4) + d->nseq
                                           : (int64_t)d->batch * ceil_div(bp->cps, 4)) *
                              d->nheads * ceil_div(d->headdim, kPGroup);
        if (walks < 256) bp->state_chunks = 1;
    }
    if (tun && tun->bwd_state_chunks) bp->state_chunks = tun->bwd_state_chunks;
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
    if (bp->state_chunks == 4) {
        // The chunk-state walks carry the state through each four-chunk
        // span: per chunk the span-local part, per span the whole (passed
        // across spans), so the pass walks a quarter of the slots.
        bp->nspan4s = d->nseq > 0 ? bp->nspan4 : (int64_t)d->batch * ceil_div(bp->cps, 4);
        const size_t st4 = (size_t)bp->nspan4s * d->nheads * d->headdim * d->d_state * esz;
        const size_t dc4 = (size_t)bp->nspan4s * d->nheads * sizeof(float);
        bp->off_ta = off;
        off = align_up(off + st4);
        bp->off_ea = off;
        off = align_up(off + dc4);
        bp->off_tb = off;
        off = align_up(off + st4);
        bp->off_eb = off;
        off = align_up(off + dc4);
    }
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

// ssd_fwd_noalloc's scratch: what ssd_fwd takes from its workspace (the
// header, span states and decays, and the varlen span table) in one fixed
// device array.  Each GPU the library runs on holds its own copy until the
// process ends.  In host code its name is only a stand-in: the device
// address comes from hipGetSymbolAddress, once per device.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of this device's scratch array (nullptr on failure).
void* scratch_address(int dev) {
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int ssd_abi_version(void) { return SSD_ABI_VERSION; }

size_t ssd_fwd_workspace_bytes(const ssd_dims* dims) {
    Plan pl;
    if (make_plan(dims, nullptr, &pl) != SSD_OK) return 0;
    return pl.total;
}

const char* ssd_status_string(int status) {
    switch (status) {
        case SSD_OK: return "SSD_OK: success";
        case SSD_ERR_NULL_ARG: return "SSD_ERR_NULL_ARG: a required pointer is NULL";
        case SSD_ERR_SHAPE:
            return "SSD_ERR_SHAPE: inconsistent or out-of-range sizes, strides or tuning values";
        case SSD_ERR_DTYPE: return "SSD_ERR_DTYPE: unknown dtype code";
        case SSD_ERR_ALIGN: return "SSD_ERR_ALIGN: pointer or stride not 16-byte aligned";
        case SSD_ERR_UNSUPPORTED:
            return "SSD_ERR_UNSUPPORTED: chunk_size or d_state not built into this library";
        case SSD_ERR_WORKSPACE: return "SSD_ERR_WORKSPACE: workspace missing or too small";
        case SSD_ERR_HIP: return "SSD_ERR_HIP: a HIP runtime call or kernel launch failed";
        case SSD_ERR_CU_SEQLENS:
            return "SSD_ERR_CU_SEQLENS: cu_seqlens not 0..L and non-decreasing";
        case SSD_ERR_OVERLAP:
            return "SSD_ERR_OVERLAP: state buffers overlap without being the same buffer";
        case SSD_ERR_SCRATCH:
            return "SSD_ERR_SCRATCH: the problem needs more scratch than ssd_fwd_noalloc's "
                   "fixed buffer (ssd_fwd_noalloc_max_bytes)";
    }
    return "unknown ssd status";
}

int ssd_fwd_plan(const ssd_dims* dims, const ssd_tuning* tuning, ssd_plan_info* out) {
    Plan pl;
    const int st = make_plan(dims, tuning, &pl);
    if (st != SSD_OK) return st;
    if (!out) return SSD_ERR_NULL_ARG;
    memset(out, 0, sizeof(*out));
    out->chunks_per_span = pl.K;
    out->col_groups = pl.npg;
    out->nspan = pl.nspan;
    out->workspace_bytes = pl.total;
    out->fused_pass = pl.fuse;
    out->heads_per_wg = pl.hg_scan;
    out->heads_per_state_wg = pl.hg_state;
    out->cols_per_wave = pl.hw_npb ? 16 * pl.hw_npb : 16;
    out->head_wave = pl.hw_npb ? 1 : 0;
    out->state_bytes = (dims->dtype == SSD_BF16 && !pl.state_f32) ? 2 : 4;
    BPlan bp;
    if (make_bwd_plan(dims, tuning, &bp) == SSD_OK) {
        out->bwd_workspace_bytes = bp.total;
        out->bwd_heads_per_wg = bp.hs;
        out->bwd_head_subsets = bp.nsub;
        out->bwd_state_chunks = bp.state_chunks;
    }
    return SSD_OK;
}

int ssd_fwd(const ssd_dims* dims, const ssd_layout* layout, const void* x, const void* d_raw,
            float d_init, const void* B, const void* C, const float* init_state,
            const int32_t* cu_seqlens, int32_t reverse, void* y, float* final_state,
            void* workspace, size_t workspace_bytes, void* stream) {
    return ssd_fwd_ex(SSD_STAGE_ALL, dims, nullptr, layout, x, d_raw, d_init, B, C, init_state,
                      cu_seqlens, reverse, y, final_state, workspace, workspace_bytes, stream);
}

// The forward call.  With rev_ws, the state stage forms both directions' span
// states in one launch: the reverse pass's into rev_ws, a workspace of the
// same plan (only whole spans in batch mode; the caller checks).
static int fwd_impl(uint32_t mask, const ssd_dims* dims, const ssd_tuning* tuning,
                    const ssd_layout* layout, const void* x, const void* d_raw, float d_init,
                    const void* B, const void* C, const float* init_state,
                    const int32_t* cu_seqlens, int32_t reverse, void* y, float* final_state,
                    void* workspace, size_t workspace_bytes, void* stream, char* rev_ws) {
    if (mask & ~(uint32_t)SSD_STAGE_ALL) return SSD_ERR_SHAPE;
    Plan pl;
    const int st = make_plan(dims, tuning, &pl);
    if (st != SSD_OK) return st;
    const ssd_dims& d = *dims;
    const int64_t T = (int64_t)d.batch * d.seqlen;
    if (T > 0 && (!x || !d_raw || !B || !C || !y)) return SSD_ERR_NULL_ARG;
    if (d.nseq > 0 && !cu_seqlens) return SSD_ERR_NULL_ARG;
    if (d.nseq == 0 && cu_seqlens) return SSD_ERR_SHAPE;
    if (reverse != 0 && reverse != 1) return SSD_ERR_SHAPE;
    const ssd_layout lay = resolve_layout(d, layout);
    const int lc = check_layout(d, lay, false);
    if (lc != SSD_OK) return lc;
    const int64_t esz = d.dtype == SSD_BF16 ? 2 : 4;
    if (!aligned16(x) || !aligned16(B) || !aligned16(C) || !aligned16(y)) return SSD_ERR_ALIGN;
    if ((uintptr_t)d_raw % esz) return SSD_ERR_ALIGN;  // read one element per lane
    if (((uintptr_t)init_state & 3u) || ((uintptr_t)final_state & 3u)) return SSD_ERR_ALIGN;
    const int64_t S = d.nseq > 0 ? d.nseq : d.batch;
    const size_t state_bytes = (size_t)S * d.nheads * d.headdim * d.d_state * sizeof(float);
    const int alias = state_alias(init_state, final_state, state_bytes);
    if (alias < 0) return SSD_ERR_OVERLAP;
    // final_state written over init_state: only the separate pass reads each
    // initial state entry before the same thread writes its final value (the
    // fold of plans 1 and 2 reads init_state in every span's workgroup)
    if (alias > 0) pl.fuse = 0;
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
    p.ys_t = lay.y_token;
    p.ys_h = lay.y_head;
    p.xs_t = lay.x_token;
    p.xs_h = lay.x_head;
    p.ds_t = lay.d_raw_token;
    p.ds_h = lay.d_raw_head;
    p.bs_t = lay.B_token;
    p.bs_g = lay.B_group;
    p.cs_t = lay.C_token;
    p.cs_g = lay.C_group;
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
    p.state_f32 = pl.state_f32;
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
    // (plan 1 with one span per sequence: the scan folds no span state, so
    // the state stage has nothing to form)
    const bool no_state = pl.fuse == 2 || (pl.fuse == 1 && pl.sps == 1);
    if ((mask & SSD_STAGE_STATE) && !no_state) {
        if (rev_ws) {
            ssd::KParams pj = p;
            pj.hg_state = d.dtype == SSD_BF16 && (d.nheads / d.ngroups) % 2 == 0 ? 2 : 1;
            pj.rev_states = rev_ws + pl.off_states;
            pj.rev_decay = (float*)(rev_ws + pl.off_decay);
            e = ssd::launch_span_state_both(pj, d.dtype, d.d_state, s);
        } else if (pl.hw_npb) {
            e = ssd::launch_hw_state(p, d.d_state, s);
        } else {
            // Plan 1: the last span of each sequence is left out (the scan
            // forms the final state itself and folds only earlier spans).
            ssd::KParams ps = p;
            if (pl.fuse == 1 && d.nseq == 0 && pl.sps > 1) {
                ps.chain_spans = pl.sps - 1;
                ps.nspan = (int64_t)d.batch * ps.chain_spans;
            }
            e = ssd::launch_span_state(ps, d.dtype, d.d_state, s);
        }
        if (e != hipSuccess) return SSD_ERR_HIP;
    }
    if ((mask & SSD_STAGE_PASS) && !pl.fuse) {
        e = ssd::launch_state_pass(p, d.dtype, s);
        if (e != hipSuccess) return SSD_ERR_HIP;
    }
    if (mask & SSD_STAGE_SCAN) {
        if (pl.fuse == 2) {
            // the fused launch's chain words and flags start from zero
            e = ssd::launch_fused_reset(p.sync, pl.nsync, s);
            if (e != hipSuccess) return SSD_ERR_HIP;
        }
        e = pl.hw_npb ? ssd::launch_hw_scan(p, d.d_state, s)
                      : ssd::launch_span_scan(p, d.dtype, d.d_state, s);
        if (e != hipSuccess) return SSD_ERR_HIP;
    }
    return SSD_OK;
}

int ssd_fwd_ex(uint32_t mask, const ssd_dims* dims, const ssd_tuning* tuning,
               const ssd_layout* layout, const void* x, const void* d_raw, float d_init,
               const void* B, const void* C, const float* init_state, const int32_t* cu_seqlens,
               int32_t reverse, void* y, float* final_state, void* workspace,
               size_t workspace_bytes, void* stream) {
    return fwd_impl(mask, dims, tuning, layout, x, d_raw, d_init, B, C, init_state, cu_seqlens,
                    reverse, y, final_state, workspace, workspace_bytes, stream, nullptr);
}

size_t ssd_fwd_bidir_workspace_bytes(const ssd_dims* dims) {
    Plan pl;
    if (make_plan(dims, nullptr, &pl) != SSD_OK) return 0;
    return 2 * align_up(pl.total);
}

int ssd_fwd_bidir(const ssd_dims* dims, const ssd_tuning* tuning, const ssd_layout* layout,
                  const void* x, const void* d_raw, float d_init, const void* B, const void* C,
                  const float* init_fwd, const float* init_rev, void* y_fwd, void* y_rev,
                  float* final_fwd, float* final_rev, void* workspace, size_t workspace_bytes,
                  void* stream) {
    Plan pl;
    const int st = make_plan(dims, tuning, &pl);
    if (st != SSD_OK) return st;
    if (dims->nseq > 0) return SSD_ERR_SHAPE;  // batch mode only
    const size_t half = align_up(pl.total);
    if (half > 0 && (!workspace || workspace_bytes < 2 * half)) return SSD_ERR_WORKSPACE;
    char* const wf = (char*)workspace;
    char* const wr = half > 0 ? wf + half : nullptr;
    // both calls checked before anything is launched (an empty stage mask)
    for (int r = 0; r < 2; ++r) {
        const int c = ssd_fwd_ex(0, dims, tuning, layout, x, d_raw, d_init, B, C,
                                 r ? init_rev : init_fwd, nullptr, r, r ? y_rev : y_fwd,
                                 r ? final_rev : final_fwd, r ? wr : wf, half, stream);
        if (c != SSD_OK) return c;
    }
    // One state launch for both directions where their spans cover the same
    // tokens (whole spans) and the plan keeps a separate state stage.
    const ssd_dims& d = *dims;
    const bool joint = d.nseq == 0 && d.seqlen > 0 && pl.fuse != 2 &&
                       d.seqlen % ((int64_t)kChunk * pl.K) == 0 &&
                       (d.d_state == 16 || d.d_state == 32 || d.d_state == 64 || d.d_state == 128);
    const uint32_t rest = joint ? (uint32_t)(SSD_STAGE_ALL & ~SSD_STAGE_STATE) : (uint32_t)SSD_STAGE_ALL;
    if (joint) {
        const int c = fwd_impl(SSD_STAGE_STATE, dims, tuning, layout, x, d_raw, d_init, B, C, init_fwd,
                               nullptr, 0, y_fwd, final_fwd, wf, half, stream, wr);
        if (c != SSD_OK) return c;
    }
    for (int r = 0; r < 2; ++r) {
        const int c = ssd_fwd_ex(rest, dims, tuning, layout, x, d_raw, d_init, B, C,
                                 r ? init_rev : init_fwd, nullptr, r, r ? y_rev : y_fwd,
                                 r ? final_rev : final_fwd, r ? wr : wf, half, stream);
        if (c != SSD_OK) return c;
    }
    return SSD_OK;
}

size_t ssd_fwd_noalloc_max_bytes(void) { return kScratchBytes; }

int ssd_fwd_noalloc(const ssd_dims* dims, const ssd_layout* layout, const void* x,
                    const void* d_raw, float d_init, const void* B, const void* C,
                    const float* init_state, const int32_t* cu_seqlens, int32_t reverse, void* y,
                    float* final_state, void* stream) {
    Plan pl;
    const int st = make_plan(dims, nullptr, &pl);
    if (st != SSD_OK) return st;
    if (pl.total > kScratchBytes) return SSD_ERR_SCRATCH;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return SSD_ERR_HIP;
    void* ptr = scratch_address(dev);
    if (!ptr) return SSD_ERR_HIP;
    return ssd_fwd_ex(SSD_STAGE_ALL, dims, nullptr, layout, x, d_raw, d_init, B, C, init_state,
                      cu_seqlens, reverse, y, final_state, ptr, kScratchBytes, stream);
}

size_t ssd_bwd_workspace_bytes(const ssd_dims* dims) {
    BPlan bp;
    if (make_bwd_plan(dims, nullptr, &bp) != SSD_OK) return 0;
    return bp.total;
}

int ssd_bwd(const ssd_dims* dims, const ssd_layout* layout, const void* x, const void* d_raw,
            float d_init, const void* B, const void* C, const float* init_state,
            const int32_t* cu_seqlens, int32_t reverse, const void* y, const void* dy,
            const float* d_final, void* dx, void* dd_raw, void* dB, void* dC,
            float* dinit_state, float* dd_init, void* workspace, size_t workspace_bytes,
            void* stream) {
    return ssd_bwd_ex(dims, nullptr, layout, x, d_raw, d_init, B, C, init_state, cu_seqlens,
                      reverse, y, dy, d_final, dx, dd_raw, dB, dC, dinit_state, dd_init, workspace,
                      workspace_bytes, stream);
}

int ssd_bwd_ex(const ssd_dims* dims, const ssd_tuning* tuning, const ssd_layout* layout,
               const void* x, const void* d_raw, float d_init, const void* B, const void* C,
               const float* init_state, const int32_t* cu_seqlens, int32_t reverse,
               const void* y, const void* dy, const float* d_final, void* dx, void* dd_raw,
               void* dB, void* dC, float* dinit_state, float* dd_init, void* workspace,
               size_t workspace_bytes, void* stream) {
    (void)y;  // not read: every gradient is formed from the inputs and the states
    BPlan bp;
    const int st = make_bwd_plan(dims, tuning, &bp);
    if (st != SSD_OK) return st;
    const ssd_dims& d = *dims;
    const int64_t T = (int64_t)d.batch * d.seqlen;
    if (T > 0 && (!x || !d_raw || !B || !C || !dy || !dx || !dd_raw || !dB || !dC))
        return SSD_ERR_NULL_ARG;
    if (d.nseq > 0 && !cu_seqlens) return SSD_ERR_NULL_ARG;
    if (d.nseq == 0 && cu_seqlens) return SSD_ERR_SHAPE;
    if (reverse != 0 && reverse != 1) return SSD_ERR_SHAPE;
    const ssd_layout lay = resolve_layout(d, layout);
    const int lc = check_layout(d, lay, true);
    if (lc != SSD_OK) return lc;
    const int64_t esz = d.dtype == SSD_BF16 ? 2 : 4;
    if (!aligned16(x) || !aligned16(B) || !aligned16(C) || !aligned16(dy) || !aligned16(dx) ||
        !aligned16(dB) || !aligned16(dC))
        return SSD_ERR_ALIGN;
    if (((uintptr_t)d_raw % esz) || ((uintptr_t)dd_raw % esz)) return SSD_ERR_ALIGN;
    if (((uintptr_t)init_state & 3u) || ((uintptr_t)d_final & 3u) || ((uintptr_t)dinit_state & 3u) ||
        ((uintptr_t)dd_init & 3u))
        return SSD_ERR_ALIGN;
    const int64_t S = d.nseq > 0 ? d.nseq : d.batch;
    const size_t state_bytes = (size_t)S * d.nheads * d.headdim * d.d_state * sizeof(float);
    // the output-gradient pass reads each d_final entry before the same
    // thread writes its dinit_state entry, so the two may be one buffer
    if (state_alias(d_final, dinit_state, state_bytes) < 0) return SSD_ERR_OVERLAP;
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
    pa.xs_t = lay.x_token;
    pa.xs_h = lay.x_head;
    pa.ds_t = lay.d_raw_token;
    pa.ds_h = lay.d_raw_head;
    pa.bs_t = lay.B_token;
    pa.bs_g = lay.B_group;
    pa.cs_t = lay.C_token;
    pa.cs_g = lay.C_group;
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
    pg.xs_t = lay.dy_token;
    pg.xs_h = lay.dy_head;
    pg.B = C;
    pg.bs_t = lay.C_token;
    pg.bs_g = lay.C_group;
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
    if (bp.state_chunks == 4) {
        if (d.nseq > 0) {
            e = ssd::launch_span_table(cu_seqlens, d.nseq, T, 4, bp.nspan4,
                                       (int32_t*)(ws + bp.off_cu4), (int32_t*)(ws + bp.off_spoff4),
                                       (int4*)(ws + bp.off_table4), s);
            if (e != hipSuccess) return SSD_ERR_HIP;
        }
        for (ssd::KParams* k : {&pa4, &pg4}) {
            k->K = 4;
            k->chunk_out = 1;
            // the state is carried through each span (the gradient set
            // walks it backwards); chunk slots keep the span-local parts
            k->chunk_run = 1;
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
        pg4.walk_rev = 1;
        pa4.span_states = ws + bp.off_ta;
        pa4.span_decay = (float*)(ws + bp.off_ea);
        pg4.span_states = ws + bp.off_tb;
        pg4.span_decay = (float*)(ws + bp.off_eb);
    }
    // the pass: over the chunks, or (four-chunk walks) over the spans'
    // whole states, leaving in each span slot the state entering the span
    // (the gradient of the state leaving it, walking backwards)
    ssd::KParams pas = pa, pgs = pg;
    if (bp.state_chunks == 4) {
        pas = pa4;
        pgs = pg4;
        pas.states = pa4.span_states;
        pas.decay = pa4.span_decay;
        pgs.states = pg4.span_states;
        pgs.decay = pg4.span_decay;
    }
    e = ssd::launch_span_state_pair(pa4, pg4, d.dtype, d.d_state, s);
    if (e == hipSuccess) e = ssd::launch_state_pass_pair(pas, pgs, d.dtype, s);
    if (e != hipSuccess) return SSD_ERR_HIP;

    ssd::BParams q;
    memset(&q, 0, sizeof(q));
    q.x = x;
    q.d_raw = d_raw;
    q.B = B;
    q.C = C;
    q.dy = dy;
    q.hprev = ws + bp.off_sa;
    q.gout = ws + bp.off_sb;
    if (bp.state_chunks == 4) {
        q.hspan = ws + bp.off_ta;
        q.gspan = ws + bp.off_tb;
        q.hdec = (const float*)(ws + bp.off_da);
        q.gdec = (const float*)(ws + bp.off_db);
        q.span_off4 = d.nseq > 0 ? (const int32_t*)(ws + bp.off_spoff4) : nullptr;
        q.sps4 = (int32_t)ceil_div(bp.cps, 4);
    }
    q.dx = dx;
    q.dd_raw = dd_raw;
    q.dB_part = (float*)(ws + bp.off_pb);
    q.dC_part = (float*)(ws + bp.off_pc);
    q.ddi_part = (float*)(ws + bp.off_pi);
    q.cu = pa.cu;
    q.table = pa.table;
    q.L = d.seqlen;
    q.ntok = T;
    q.xs_t = lay.x_token;
    q.xs_h = lay.x_head;
    q.gs_t = lay.dy_token;
    q.gs_h = lay.dy_head;
    q.ds_t = lay.d_raw_token;
    q.ds_h = lay.d_raw_head;
    q.bs_t = lay.B_token;
    q.bs_g = lay.B_group;
    q.cs_t = lay.C_token;
    q.cs_g = lay.C_group;
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
