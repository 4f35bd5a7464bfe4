// Internal declarations shared by the C-ABI layer (ssd_api.hip) and the
// kernels (ssd_kernels.hip).  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ssd {

constexpr int kChunk = 64;     // tokens per chunk (one wavefront of lanes)
constexpr int kWaves = 4;      // wavefronts per workgroup in the span kernels
constexpr int kThreads = 256;  // kWaves * 64
constexpr int kPGroup = 64;    // headdim columns per workgroup (16 per wave)
constexpr int kXcds = 8;       // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr int kXcdCus = 32;    // MI355X: 32 CUs per XCD

// n / d for 0 <= n < 2^31 as a multiply-high, an add and a shift: with
// l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1, the quotient is
// (mulhi(n, m) + n) >> l (Granlund and Montgomery, "Division by Invariant
// Integers using Multiplication", PLDI 1994, section 4; for such n the sum
// stays below 2^32).  A launch's divisors are fixed, so its launcher picks m
// and l on the host and the kernels' index decode needs no division.
struct FastDiv {
    uint32_t m, l;
};
inline FastDiv make_fastdiv(uint32_t d) {
    FastDiv f{1u, 0u};  // d <= 1: n itself
    if (d <= 1) return f;
    while ((1ull << f.l) < d) ++f.l;
    f.m = (uint32_t)(((1ull << 32) * ((1ull << f.l) - d)) / d + 1);
    return f;
}
__device__ __forceinline__ uint32_t fdiv(uint32_t n, FastDiv f) {
    return (__umulhi(n, f.m) + n) >> f.l;
}

// A span launch's grid decode, filled in by its launcher (set_decode) from
// the sizes below and the launch's heads per workgroup.
struct Decode {
    int64_t nreal;   // work items: span slots x head groups x column groups
    int64_t per;     // work items per XCD, ceil(nreal / kXcds)
    int32_t ngrp;    // head groups of the launch's heads per workgroup
    int32_t nchain;  // chains: batch x ngrp x npg
    int32_t cpx;     // chains per XCD, nchain / kXcds
    FastDiv by_npg, by_ngrp, by_cpx, by_sps, by_batch, by_hpg;  // hpg = H / G
    FastDiv by_ev, by_h, by_nb;  // state pass: entry vectors per state, H, N / 16
};

// Everything the kernels need, passed by value.
struct KParams {
    const void* x;          // [b, L, H, P]
    const void* d_raw;      // [b, L, H]
    const void* B;          // [b, L, G, N]
    const void* C;          // [b, L, G, N]
    void* y;                // strided output
    const float* init;      // [S, H, N, P] or null
    float* final_state;     // [S, H, N, P] or null
    void* states;           // [nspan][H][P][N] span states / incoming states,
                            // stored in the input type (accumulated in fp32)
    float* decay;           // [nspan][H] span decay products
    const int32_t* cu;      // sanitized cu_seqlens [nseq+1] (varlen) or null
    const int32_t* span_off;// [nseq+1] first span of each sequence (varlen)
    const int4* table;      // [nspan] {seq, chunk0, nchunks, 0} (varlen)
    int64_t L;              // tokens per batch row
    int64_t ys_t, ys_h;     // y strides (elements)
    int64_t xs_t, xs_h;     // x strides (elements): token, head (H*P and P
                            // for a contiguous x)
    int64_t ds_t, ds_h;     // d_raw strides: token, head (H and 1)
    int64_t bs_t, bs_g;     // B strides: token, group (G*N and N)
    int64_t cs_t, cs_g;     // C strides: token, group
    int64_t nspan;          // span slots (grid extent)
    int32_t batch, H, P, G, N;
    int32_t nseq;           // 0 = batch mode
    int32_t K;              // chunks per span
    int32_t sps;            // spans per sequence (batch mode)
    int32_t npg;            // headdim column groups of kPGroup
    int32_t hg_state;       // heads per span_state workgroup (divides H/G)
    int32_t hg_scan;        // heads per span_scan workgroup (divides H/G)
    int32_t reverse;
    int32_t fuse_pass;      // batch mode, few spans per sequence.  1: span_scan
                            // forms each span's incoming state from the span
                            // states itself and writes final_state (no
                            // state_pass).  2: one fused launch does all.
    int32_t hw_npb;         // head-wave kernels: 16-column blocks per wave (2 or
                            // 4); 0 = span kernels
    uint32_t* sync;         // workspace header; for fuse_pass 2 followed by one
                            // 64-bit ticket/epoch word per chain and one flag
                            // per workgroup
    int32_t wmode;          // state-update weights of span_state: 0 the
                            // forward's e^{cs_last - cs_s} d_s, 1 e^{cs_s}
                            // (the backward's output-gradient state)
    int32_t pass_desc;      // state_pass walks each sequence's spans from
                            // its last to its first
    int32_t chunk_out;      // span_state, K <= 4: store the local state and
                            // decay of every chunk of the span instead of the
                            // span's, in slot seq * chunks-per-sequence +
                            // chunk (batch mode) or chunk_slot[seq] + chunk
                            // (varlen)
    const int32_t* chunk_slot;  // (varlen, chunk_out) first chunk slot of each
                                // sequence
    int32_t chunk_run;      // (chunk_out) the state is carried through the
                            // span: chunk c's slot gets the span-local state
                            // entering it (the chunks walked before it) and
                            // its decay slot their decay product; the span's
                            // whole local state and decay product go to
                            // span_states / span_decay at slot span
    int32_t walk_rev;       // (chunk_run) walk the span's chunks from its last
                            // to its first (the output-gradient state, which
                            // flows against the processing order)
    void* span_states;      // (chunk_run) [nspan][H][P][N], input type
    float* span_decay;      // (chunk_run) [nspan][H]
    void* rev_states;       // (both directions) the reverse pass's span states
    float* rev_decay;       // ... and span decays, same layout as states / decay
    int32_t state_f32;      // span states stored in float32 whatever the input
                            // type (span kernels, plans 0 and 1)
    int32_t chain_spans;    // (state launch of plan 1, batch mode) spans per
                            // sequence it forms: the first sps - 1 (no scan
                            // folds the last one's state); 0 = all
    float d_init;
    Decode dc;              // set by the launcher of each span kernel
};

// The decode of a launch with hg heads per workgroup (the host keeps the
// work items below 2^31 and G dividing H).
inline void set_decode(KParams& p, int hg) {
    Decode& d = p.dc;
    d.ngrp = (p.H + hg - 1) / hg;
    d.nreal = p.nspan * d.ngrp * p.npg;
    d.per = (d.nreal + kXcds - 1) / kXcds;
    d.nchain = p.batch * d.ngrp * p.npg;
    d.cpx = d.nchain / kXcds;
    d.by_npg = make_fastdiv((uint32_t)p.npg);
    d.by_ngrp = make_fastdiv((uint32_t)d.ngrp);
    d.by_cpx = make_fastdiv((uint32_t)d.cpx);
    d.by_sps = make_fastdiv((uint32_t)p.sps);
    d.by_batch = make_fastdiv((uint32_t)p.batch);
    d.by_hpg = make_fastdiv((uint32_t)(p.G > 0 ? p.H / p.G : 1));
}

// The decode of a state pass moving V state entries per thread.
inline void set_pass_decode(KParams& p, int V) {
    p.dc.by_ev = make_fastdiv((uint32_t)((int64_t)p.P * p.N / V));
    p.dc.by_h = make_fastdiv((uint32_t)p.H);
    p.dc.by_nb = make_fastdiv((uint32_t)(p.N / 16));
}

// Backward pass (ssd_bwd_kernels.hip): one workgroup per (chunk, B/C
// group, subset of hs heads of the group); headdim <= 64.
struct BParams {
    const void* x;          // [b, L, H, P] (strides xs_t, xs_h; dx shares them)
    const void* d_raw;      // [b, L, H]
    const void* B;          // [b, L, G, N]
    const void* C;
    const void* dy;         // dL/dy (strides gs_t, gs_h)
    const void* hprev;      // [nchunk][H][P*N] state entering each chunk
    const void* gout;       // [nchunk][H][P*N] dL/d(state leaving each chunk)
    // With carried chunk states (hspan non-null) hprev and gout hold only
    // the span-local parts: the state entering chunk c is hdec[c] times the
    // state entering its four-chunk span (hspan) plus hprev[c], and the
    // gradient of the state leaving it gdec[c] times the gradient of the
    // state leaving the span (gspan) plus gout[c].
    const void* hspan;      // [nspan4][H][P*N] or null
    const void* gspan;      // [nspan4][H][P*N]
    const float* hdec;      // [nchunk][H]
    const float* gdec;      // [nchunk][H]
    const int32_t* span_off4;  // (varlen) first four-chunk span of each sequence
    int32_t sps4;           // (batch mode) four-chunk spans per sequence
    void* dx;               // [b, L, H, P], strided like x
    void* dd_raw;           // [b, L, H], strided like d_raw
    float* dB_part;         // [nsub][ntok][G][N] per head subset
    float* dC_part;
    float* ddi_part;        // [nchunk * G * nsub] per workgroup
    const int32_t* cu;      // sanitized cu_seqlens (varlen) or null
    const int4* table;      // [nchunk] {seq, chunk, 1, 0} (varlen)
    int64_t L, ntok;        // tokens per batch row, b * L
    int64_t xs_t, xs_h, gs_t, gs_h;
    int64_t ds_t, ds_h;     // d_raw (and dd_raw) strides: token, head
    int64_t bs_t, bs_g;     // B (and dB) strides: token, group
    int64_t cs_t, cs_g;     // C (and dC) strides: token, group
    int64_t nchunk;         // chunk slots (grid extent / G / nsub)
    int32_t batch, H, P, G, N;
    int32_t nseq;
    int32_t cps;            // chunks per sequence (batch mode)
    int32_t nsub, hs;       // head subsets per group, heads per subset
    int32_t reverse;
    float d_init;
    FastDiv by_nsub, by_G, by_cps, by_npg;  // set by the gradient launcher
};
constexpr int kBwdMaxHeads = 64;  // heads one backward workgroup carries at most
bool bwd_supported(int dtype, int N);
hipError_t launch_bwd_chunk(const BParams& p, int dtype, hipStream_t s);
hipError_t launch_bwd_reduce(const BParams& p, int dtype, void* dB, void* dC, float* dd_init,
                             hipStream_t s);

// Zero the fused launch's chain words and flags (and the header's timeout
// count) before it runs, so each fused call starts from a known state.
hipError_t launch_fused_reset(uint32_t* sync, int64_t nwords, hipStream_t s);

// Most spans per sequence for which span_scan forms the incoming states
// itself (each workgroup folds all earlier spans of its sequence).
constexpr int kFuseSpans = 16;

// The workspace header: its first 256 bytes, of which word 2 counts the
// fused launch's bounded flag waits that ran out.  The fused launch keeps
// its ticket/epoch words and flags after it; a reset kernel zeroes them
// (and word 2) before every fused launch.
constexpr int kSyncTimeouts = 2;
constexpr int kSyncHeader = 64;
// Polls (each followed by a 64-cycle sleep) one workgroup spends at most
// waiting for the flags of the earlier spans of its sequence.
constexpr uint32_t kSpinBudget = 1u << 20;

// Launchers (ssd_kernels.hip).  Each returns hipSuccess or the launch error.
hipError_t launch_span_table(const int32_t* cu_raw, int32_t nseq, int64_t T,
                             int32_t K, int64_t nspan, int32_t* cu_san,
                             int32_t* span_off, int4* table, hipStream_t s);
hipError_t launch_span_state(const KParams& p, int dtype, int N, hipStream_t s);
hipError_t launch_span_state_both(const KParams& p, int dtype, int N, hipStream_t s);
hipError_t launch_state_pass(const KParams& p, int dtype, hipStream_t s);
hipError_t launch_span_scan(const KParams& p, int dtype, int N, hipStream_t s);
// The backward pass's two chunk-state passes (pa: kModeState on (B, x), pb:
// weights e^{cs} on (C, dy); same sizes, one head per workgroup) and their two
// state passes, each pair in one launch.
hipError_t launch_span_state_pair(const KParams& pa, const KParams& pb, int dtype, int N,
                                  hipStream_t s);
hipError_t launch_state_pass_pair(const KParams& pa, const KParams& pb, int dtype, hipStream_t s);

// Head-wave kernels (ssd_hw_kernels.hip): bf16, d_state 64 or 128; hg heads
// per workgroup (1, 2, 4), npb 16-column blocks per wave (2, 4).
bool hw_supported(int dtype, int N, int hg, int npb);
size_t hw_lds_bytes(int N, int hg, int npb, bool scan);
hipError_t launch_hw_state(const KParams& p, int N, hipStream_t s);
hipError_t launch_hw_scan(const KParams& p, int N, hipStream_t s);

// Most heads one span workgroup can carry for this d_state.
int span_max_heads(int dtype, int N, bool scan);

// LDS bytes one span workgroup uses for (dtype, N, scan); 0 = not built.
size_t span_lds_bytes(int dtype, int N, bool scan);

}  // namespace ssd
