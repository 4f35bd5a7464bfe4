// HIP kernels for the Mamba-2 SSD chunked scan on gfx950 (MI355X).
//
// The scan per head ("Mamba-2架构与LaCT并行计算技术解析", §1.1):
//   d_t = softplus(d_raw_t + d_init),  H_t = exp(-d_t) H_{t-1} + d_t B_t^T X_t,
//   y_t = C_t H_t.
// It is evaluated in the chunked semiseparable form of "长序列 Mamba 多卡训练，
// 算力和显存怎么同时省", §一: with cs the within-chunk cumulative sum of -d,
//   y_t = sum_{s<=t in chunk} (C_t.B_s) e^{cs_t-cs_s} d_s X_s + e^{cs_t} C_t Hprev
//   H_end = e^{cs_last} Hprev + sum_s B_s^T (e^{cs_last-cs_s} d_s X_s)
// and the state crosses chunk borders as (decay, state) pairs, the combine
// that the Mamba context-parallel scheme of "揭秘MindSpeed-LLM多潜在注意力（MLA）
// 与Mamba上下文并行实现原理", §三.2, applies across devices.
//
// Kernels (one launch each, all on the caller's stream):
//   span_table  (packed batches only) one workgroup turns cu_seqlens into a
//               table of spans; a span is up to K consecutive 64-token chunks
//               of one sequence.
//   span_state  per (span, group of heads, 64 headdim columns): the span's
//               local state S = sum over its chunks, with the chunk decays,
//               of B^T (w * X) on MFMA, and the span decay product.
//   state_pass  per (sequence, head, 4 state entries): walks the spans in
//               order, H <- decay * H + S, overwriting each S with the state
//               entering its span; writes final_state.
//   span_scan   per (span, group of heads, 64 columns): starts from the
//               incoming states and, chunk by chunk, forms C B^T once for all
//               heads of the group, applies each head's causal decay mask,
//               adds the C Hprev term and writes y, then advances the states
//               (kept in MFMA accumulators) to the next chunk.
// Inside a span the states stay on chip; only span borders go through HBM.
// B and C are shared by all heads of a group (ngroups heads per group), so a
// workgroup stages them, and forms C B^T, once per chunk for all its heads.
//
// MFMA tiling (v_mfma_f32_16x16x32_bf16; fp32 inputs use 8 x 16x16x4_f32):
// lane l of a wave holds operand row/column l%16 and eight K values chosen by
// l/16; the 16x16 fp32 result holds rows 4*(l/16)+i, column l%16.  A result
// tile pair therefore already is an operand fragment (K = the tile rows), so
// C B^T feeds the intra-chunk product and the state feeds C Hprev with no
// data movement.  Any K order works as long as both operands agree.  Outputs
// are formed transposed (y^T = X^T L^T + H^T C^T) so each lane holds four
// consecutive headdim values of one token and stores them in one access.
#include "ssd_device.h"

namespace ssd {
namespace {

// Compile-time shape of one span workgroup: HG heads sharing one B/C group,
// one quad of 4 waves per head, each wave one 16-column block of the 64
// headdim columns of the group.
template <typename T, int N, int HG>
struct Cfg {
    static constexpr int TH = kThreads * HG;     // threads per workgroup
    static constexpr int NW = TH / 64;           // waves per workgroup
    static constexpr int NB = N / 16;            // 16-row blocks of the state
    static constexpr int KN = (N + 31) / 32;     // K=32 steps over the state dim
    static constexpr int EPU = 16 / sizeof(T);   // elements per 16-byte unit
    static constexpr int XU = kPGroup / EPU;     // 16-byte units per X row
    static constexpr int BU = N / EPU;           // 16-byte units per B / C row
};

// Heads (quads) per workgroup: up to 2 (8 waves), one for the scan when a
// state row is wider than 256 bytes (its per-wave registers exceed 256).
constexpr int heads_state(int N, int esz) { return 2; }
constexpr int heads_scan(int N, int esz) { return N * esz <= (esz == 2 ? 256 : 128) ? 2 : 1; }


// Fragment slots of the masked C B^T, the B operand of y^T += X^T L^T:
// (tb, kk) -> tb=0: 0, tb=1: 1, tb=2: 2+kk, tb=3: 4+kk.
__device__ __forceinline__ constexpr int lslot(int tb, int kk) {
    return tb == 0 ? 0 : (tb == 1 ? 1 : (tb == 2 ? 2 + kk : 4 + kk));
}


// v itself, as an expression that depends on the tag's type: uses of v
// inside `if constexpr` on the tag are then checked only where taken.
template <typename Tag, typename V>
__device__ __forceinline__ const V& dep_on(Tag, const V& v) { return v; }

// LDS of one span workgroup.  X and B tiles are double-buffered: chunk
// c+1's fill one buffer while chunk c is computed from the other.  The C tile
// has one buffer, refilled as soon as the step's C reads are done.  Decay
// factors are formed four chunks at a time (one chunk per wave of a quad)
// from d_raw loaded one such batch ahead.
template <typename T, int N, int HG, bool SCAN, bool BOTH = false>
struct __attribute__((aligned(16))) Smem {
    using X4 = typename Vec<T>::x4;
    T xs[2][HG][kChunk * kPGroup];      // X of every head, this group's 64 columns
    T bs[2][kChunk * N];                // B
    T cs[SCAN ? kChunk * N : 1];        // C (scan)
    // masked C B^T per head (scan): fragment slot, half, lane -- each half a
    // contiguous run of 64 8-byte (bf16) values, so writes and reads of one
    // half never share a bank
    X4 lf[SCAN ? HG : 1][SCAN ? 6 : 1][2][SCAN ? 64 : 1];
    // chunk 4b + w of the current batch b, per head (a state pass keeps only
    // what its update needs)
    std::conditional_t<SCAN, Decay, std::conditional_t<BOTH, DecayS2, DecayS>> dec[kWaves][HG];
    __attribute__((aligned(16))) uint32_t dr[2][kWaves][HG][kChunk];  // d_raw of a batch, per lane
    uint32_t ticket, epoch;  // fused kernel: this workgroup's ticket and epoch
};


// One 16x16 tile (t-block TB, s-block SB) of C B^T for head q: rows
// s = 16*SB + 4g + i, column t = 16*TB + l16 of the MFMA result, times the
// head's decay mask, rounded, written as half SB&1 of q's fragment slot.
template <int TB, int SB, typename T, int N, int HG, bool SCAN>
__device__ __forceinline__ void mask_tile(Smem<T, N, HG, SCAN>& sm, const Decay& D, int q,
                                          int lane,
                                          const typename Vec<T>::x8 (&bf)[Cfg<T, N, HG>::KN],
                                          const typename Vec<T>::x8 (&cf)[Cfg<T, N, HG>::KN]) {
    using X4 = typename Vec<T>::x4;
    constexpr int KN = Cfg<T, N, HG>::KN;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KN; ++kk) acc = mma(bf[kk], cf[kk], acc);
    const int l16 = lane & 15, s0 = 16 * SB + 4 * (lane >> 4);
    X4 v;
    if constexpr (TB > SB) {  // off-diagonal: no exponentials
        const f32x4 fa = *(const f32x4*)&D.fa[s0];
        const float f = D.fm[TB * (TB - 1) / 2 + SB] * D.fb[16 * TB + l16];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = cvt<T>(acc[i] * (fa[i] * f));
    } else {  // diagonal: mask s <= t before the exponential
        const int t = 16 * TB + l16;
        const float cst = D.cs2[t];
        const f32x4 css = *(const f32x4*)&D.cs2[s0];
        const f32x4 dts = *(const f32x4*)&D.dt[s0];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool causal = (s0 + i) <= t;
            const float e = fexp2(causal ? cst - css[i] : -INFINITY);
            v[i] = cvt<T>(causal ? acc[i] * e * dts[i] : 0.f);
        }
    }
    if constexpr (SCAN) sm.lf[q][lslot(TB, SB >> 1)][SB & 1][lane] = v;
}

// Register budget: 2 waves per SIMD (256 VGPRs) where the kernel fits in
// them -- two 4-wave workgroups per CU, or one 8-wave one (an 8-wave
// workgroup needs two waves per SIMD to fit a CU at all).  The variants whose
// fragments and state need more (bf16 d_state 256; fp32 d_state 128 states,
// fp32 d_state >= 64 scans) get one wave per SIMD and up to 512 VGPRs.
enum { kModeState = 0, kModeScan = 1, kModeFused = 2, kModeStateGrad = 3, kModeStateBoth = 4 };
constexpr bool is_state(int mode) {
    return mode == kModeState || mode == kModeStateGrad || mode == kModeStateBoth;
}
template <typename T, int N, int HG, int MODE>
constexpr int span_occupancy() {
    if (HG != 1) return 2;
    if (sizeof(T) == 2) return N <= 128 ? 2 : 1;
    return (is_state(MODE) ? N <= 64 : N <= 32) ? 2 : 1;
}

// Accesses coherent across the whole device (agent scope, all XCDs): the
// span states, decays and flags that workgroups of one launch hand to each
// other.  Stores write through to the point of coherence; loads read from it.
__device__ __forceinline__ void coherent_store32(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t coherent_load32(const uint32_t* p) {
    return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void coherent_store64(void* p, uint64_t v) {
    __hip_atomic_store((uint64_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t coherent_load64(const void* p) {
    return __hip_atomic_load((uint64_t*)const_cast<void*>(p), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}
// Four state entries, stored in the input type (8 or 16 bytes).
__device__ __forceinline__ void coherent_store4(bf16* p, const f32x4& v) {
    bf16x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = (bf16)v[i];
    coherent_store64(p, __builtin_bit_cast(uint64_t, o));
}
__device__ __forceinline__ void coherent_store4(float* p, const f32x4& v) {
    coherent_store64(p, __builtin_bit_cast(uint64_t, f32x2{v[0], v[1]}));
    coherent_store64(p + 2, __builtin_bit_cast(uint64_t, f32x2{v[2], v[3]}));
}
// Four stored state entries as loaded (8 or 16 bytes), widened by widen4.
__device__ __forceinline__ bf16x4 coherent_load_raw4(const bf16* p) {
    return __builtin_bit_cast(bf16x4, coherent_load64(p));
}
__device__ __forceinline__ f32x4 coherent_load_raw4(const float* p) {
    const f32x2 lo = __builtin_bit_cast(f32x2, coherent_load64(p));
    const f32x2 hi = __builtin_bit_cast(f32x2, coherent_load64(p + 2));
    return f32x4{lo[0], lo[1], hi[0], hi[1]};
}
__device__ __forceinline__ bf16x4 load_raw4(const bf16* p) { return *(const bf16x4*)p; }
__device__ __forceinline__ f32x4 load_raw4(const float* p) { return *(const f32x4*)p; }
__device__ __forceinline__ f32x4 widen4(const bf16x4& v) {
    return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
__device__ __forceinline__ f32x4 widen4(const f32x4& v) { return v; }
// Wait until every memory access this wave issued has completed (stores
// acknowledged by the point of coherence); the compiler moves no memory
// access across it.
__device__ __forceinline__ void drain_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Span workgroups.
//  kModeState  the span's local state from a zero state, and its decay
//              product (span_state).
//  kModeStateGrad  the same with weights e^{cs_s} in place of
//              e^{cs_last - cs_s} d_s: on (C, dy) the backward pass's
//              chunk-local output-gradient state.
//  kModeScan   y from the state entering the span: as state_pass left it,
//              or (fuse_pass 1) folded here from the span states of the
//              earlier spans of the sequence, with the last span then also
//              writing final_state (span_scan).
//  kModeFused  both in one launch (fuse_pass 2, batch mode): workgroups
//              take tickets in span order; each forms its span's local state
//              and publishes it with a flag, waits for the flags of the
//              earlier spans of its sequence (all held by earlier tickets, so
//              running or done), folds their states into the state entering
//              its span, and writes y.  The last span of a sequence skips the
//              local state (no later span reads it) and writes final_state.
template <typename T, int N, int HG, int MODE>
__device__ __forceinline__ void span_body(const KParams& p, int64_t blk,
                                          Smem<T, N, HG, !is_state(MODE), MODE == kModeStateBoth>& sm) {
    using Cf = Cfg<T, N, HG>;
    using X8 = typename Vec<T>::x8;
    using X4 = typename Vec<T>::x4;
    constexpr int NB = Cf::NB, KN = Cf::KN, EPU = Cf::EPU;
    constexpr int W = 16 / EPU;               // 16-byte units per block row
    constexpr int XI = 4 * W, BI = NB * W;    // load instructions per X / B / C tile
    constexpr bool SCANL = !is_state(MODE);  // LDS holds the scan buffers

    const int hg = is_state(MODE) ? p.hg_state : p.hg_scan;
    const Decode& dc = p.dc;  // this launch's decode (divisions by its sizes)
    const int ngrp = dc.ngrp;
    const int64_t nreal = dc.nreal;
    const int tid = threadIdx.x;
    int64_t logical;
    uint32_t epoch = 0;
    if constexpr (MODE == kModeFused) {
        // Workgroup b serves chain b / sps (one sequence, head group and
        // column group) and takes the next span of that chain from the
        // chain's 64-bit header word: the low half counts the chain's
        // workgroups so far, so a workgroup waits only for spans already
        // held by running ones; the high half is the chain's launch epoch,
        // which tags its flags.  The chain's last workgroup resets the count
        // and advances the epoch for the next launch.
        const int64_t per_seq = (int64_t)ngrp * p.npg;
        const int64_t chain = blk / p.sps;
        if (tid == 0) {
            const uint64_t te = __hip_atomic_fetch_add((uint64_t*)(p.sync + kSyncHeader) + chain, 1ull,
                                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const uint32_t t = (uint32_t)te, e = (uint32_t)(te >> 32);
            if (t == (uint32_t)(p.sps - 1))
                coherent_store64((uint64_t*)(p.sync + kSyncHeader) + chain, (uint64_t)(e + 1) << 32);
            sm.ticket = t;
            sm.epoch = e + 1;
        }
        block_sync();
        // (a header not zero-filled before the first launch still maps every
        // ticket to a span in range)
        const int64_t kin = sm.ticket % (uint32_t)p.sps;
        epoch = sm.epoch;
        const int64_t seq = chain / per_seq;
        logical = (seq * p.sps + kin) * per_seq + (chain - seq * per_seq);
    } else {
        // XCD-aware order: consecutive logical blocks (same span, neighbouring
        // head groups, which share B and C) land on the same XCD and its L2.
        const int64_t bid = blk;
        logical = (bid % kXcds) * dc.per + bid / kXcds;
        if (logical >= nreal) return;
    }
    // (the host keeps span x head group x column group below 2^31, so the
    // decode divides in 32 bits)
    int pg, hgi;
    uint32_t span32;
    const uint32_t nchain = (uint32_t)dc.nchain;
    if ((MODE == kModeScan || (MODE == kModeState && !p.chunk_out)) && p.fuse_pass == 1 &&
        !p.nseq && nchain % kXcds == 0) {
        // A scan that folds the earlier span states itself, and the state
        // launch before it: each XCD takes whole chains (sequence, head
        // group, column group), every span of them, so the fold's re-reads
        // of a chain's span states meet in one L2 (the XCD that formed them)
        // and each XCD folds the same amount.  Ranked by fold length (rank
        // 0: the last position), the workgroups are placed so that the
        // longest folds get a CU of their own: with n workgroups on an
        // XCD's c CUs (c < n <= 2c), slots j and j + c (j < n - c) share a
        // CU and slots n - c .. c - 1 run alone; the alone slots take the
        // first 2c - n ranks, and each shared CU pairs the next heaviest
        // rank with the lightest one left.
        const uint32_t S = (uint32_t)p.sps, cpx = (uint32_t)dc.cpx;
        const uint32_t SL = p.chain_spans ? (uint32_t)p.chain_spans : S;  // spans formed per chain
        const uint32_t x = (uint32_t)(blk % kXcds), slot = (uint32_t)(blk / kXcds);
        const uint32_t n = SL * cpx, c = kXcdCus;
        uint32_t rank = slot;
        if (n > c && n <= 2 * c) {
            const uint32_t np = n - c;  // CUs holding two
            if (slot >= np && slot < c) rank = slot - np;
            else if (slot < np) rank = (2 * c - n) + slot;
            else rank = n - 1 - (slot - c);
        }
        const uint32_t pr = fdiv(rank, dc.by_cpx), chain = x * cpx + (rank - pr * cpx);
        const uint32_t rest = fdiv(chain, dc.by_npg);
        pg = (int)(chain - rest * (uint32_t)p.npg);
        const uint32_t seq = fdiv(rest, dc.by_ngrp);
        hgi = (int)(rest - seq * (uint32_t)ngrp);
        span32 = seq * S + (SL - 1u - pr);
    } else {
        const uint32_t lg32 = (uint32_t)logical, rest = fdiv(lg32, dc.by_npg);
        pg = (int)(lg32 - rest * (uint32_t)p.npg);
        span32 = fdiv(rest, dc.by_ngrp);
        hgi = (int)(rest - span32 * (uint32_t)ngrp);
        if (MODE != kModeFused && !p.nseq && p.batch > 1) {
            // Interleave the sequences' spans, each odd sequence's in reverse
            // order: neighbouring logical spans (one XCD) then pair an early
            // and a late position, the later one first.  (A launch forming
            // only the first chain_spans spans of each sequence interleaves
            // those; with batch 1 its work items are those spans already.)
            const uint32_t B = (uint32_t)p.batch, S = (uint32_t)p.sps;
            const uint32_t SL = p.chain_spans ? (uint32_t)p.chain_spans : S;
            const uint32_t k = fdiv(span32, dc.by_batch), j = span32 - k * B;
            const uint32_t sq = 2u * k < SL ? B - 1u - j : j;
            span32 = sq * S + ((sq & 1u) ? SL - 1u - k : k);
        }
    }
    const int64_t span = span32;
    const int h0 = hgi * hg;
    const int nh = min(hg, p.H - h0);  // hg <= HG divides H/G: one B/C group

    int64_t start, len;
    int chunk0, nck, vseq = 0;
    if (p.nseq) {
        const int4 e = p.table[span];
        if (e.x < 0) return;
        vseq = e.x;
        start = p.cu[e.x];
        len = (int64_t)p.cu[e.x + 1] - start;
        chunk0 = e.y;
        nck = e.z;
    } else {
        const uint32_t seq = fdiv(span32, dc.by_sps);
        const int kin = (int)(span32 - seq * (uint32_t)p.sps);
        start = (int64_t)seq * p.L;
        len = p.L;
        const int64_t nch = (len + kChunk - 1) / kChunk;
        chunk0 = kin * p.K;
        nck = (int)imin(p.K, nch - chunk0);
    }
    if (nck <= 0) return;

    const int pcol0 = pg * kPGroup;
    const int pgw = min(kPGroup, p.P - pcol0);
    const int wave = wave_id(), lane = tid & 63;
    const int l16 = lane & 15, g = lane >> 4;
    const int q = wave >> 2, w4 = wave & 3;  // quad = head h0 + q; 16-column block w4
    const bool live = q < nh;                // this quad has a head
    const bool active = live && w4 * 16 < pgw;  // this wave's results are stored
    const int pb = pg * kWaves + w4;  // this wave's 16-column block of headdim
    const int h = h0 + q;

    // Token of row r of chunk c: tok0(c) + dir * r.
    const int dir = p.reverse ? -1 : 1;
    // token strides (the host keeps them <= 2^24)
    const int XS = (int)p.xs_t, BS = (int)p.bs_t, CS = (int)p.cs_t, DS = (int)p.ds_t;
    const int grp = (int)fdiv((uint32_t)h0, dc.by_hpg);  // h0 G / H
    // Every wave computes, with a valid head even in a quad without one or
    // past the headdim; only active waves store what they computed.
    const int hc = live ? h : h0;
    const T* const xg = (const T*)p.x + (int64_t)hc * p.xs_h + pcol0;
    const T* const bg = (const T*)p.B + (int64_t)grp * p.bs_g;
    const T* const cg = (const T*)p.C + (int64_t)grp * p.cs_g;
    const T* const dg = (const T*)p.d_raw + (int64_t)hc * p.ds_h;
    // Step c of the walk takes chunk ck(c) of the span: the span's chunks
    // in order, or (a reversed chunk-state walk) from its last to its first.
    // Row 0 of chunk k is token tb0 + k * dstep; its tokens left in the
    // sequence are rem0 - 64k.
    const bool wrev = is_state(MODE) && p.chunk_out && p.chunk_run && p.walk_rev;
    auto ck = [&](int c) -> int { return wrev ? nck - 1 - c : c; };
    const int64_t cj0 = (int64_t)chunk0 * kChunk;
    const int64_t tb0 = start + (p.reverse ? len - 1 - cj0 : cj0);
    const int dstep = dir * kChunk;
    const int64_t rem0 = len - cj0;
    auto tok0 = [&](int c) -> int64_t { return tb0 + (int64_t)(ck(c) * dstep); };
    auto clen_of = [&](int c) -> int { return (int)imin(kChunk, rem0 - (int64_t)ck(c) * kChunk); };
    // chunk k's row-0 pointers: base at chunk 0 plus k chunk steps
    const T* const xc0 = xg + tb0 * XS;
    const T* const bc0 = bg + tb0 * BS;
    const T* const cc0 = cg + tb0 * CS;
    const int64_t xcs = (int64_t)dstep * XS, bcs = (int64_t)dstep * BS, ccs = (int64_t)dstep * CS;
    // Step c's X tile (wave w4 loads its own 16-column block) and this
    // wave's share of the B tile.
    auto issue_xb = [&](int c, T* __restrict__ xdst, T* __restrict__ bdst) {
        const int cl = clen_of(c);
        issue_tile<W, 1, XI>(xdst, xc0 + ck(c) * xcs, dir * XS, w4 * W, cl, pgw, lane);
        issue_tile<(BI + Cf::NW - 1) / Cf::NW, Cf::NW, BI>(bdst, bc0 + ck(c) * bcs, dir * BS, wave, cl,
                                                        N, lane);
    };
    // This wave's share of chunk c's C tile (scan).
    auto issue_c = [&](int c, T* __restrict__ cdst) {
        if constexpr (SCANL)
            issue_tile<(BI + Cf::NW - 1) / Cf::NW, Cf::NW, BI>(cdst, cc0 + c * ccs, dir * CS, wave,
                                                            clen_of(c), N, lane);
    };
    // The quad head's d_raw of chunk c, one token per lane.
    auto issue_d = [&](int c, uint32_t* __restrict__ ddst) {
        const int cl = clen_of(c);
        const void* src = (const void*)(dg + (tok0(c) + dir * (lane < cl ? lane : 0)) * DS);
        auto* lds = (__attribute__((address_space(3))) void*)ddst;
        if constexpr (sizeof(T) == 2) __builtin_amdgcn_global_load_lds(src, lds, 2, 0, 0);
        else __builtin_amdgcn_global_load_lds(src, lds, 4, 0, 0);
    };

    // span within its sequence, and the sequence (batch mode; varlen never
    // folds or reads these)
    const uint32_t seq_of = p.sps > 0 ? fdiv(span32, dc.by_sps) : span32;
    const int kin = (int)(span32 - seq_of * (uint32_t)(p.sps > 0 ? p.sps : 1));
    const bool folds = MODE == kModeFused || (MODE == kModeScan && p.fuse_pass);
    const bool write_final = folds && p.final_state && kin == p.sps - 1;
    // (n, p) of this lane's entry i of state block nb, [N][P] offset
    auto np_off = [&](int nb, int i) -> int64_t {
        return (int64_t)(16 * nb + 4 * g + i) * p.P + 16 * pb + l16;
    };
    const int64_t hseq = ((int64_t)seq_of * p.H + h) * (int64_t)N * p.P;
    f32x4 Hs[NB];  // this wave's 16 columns of the state, MFMA result order
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) Hs[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    float logdec2 = 0.f;  // first wave of each quad: sum of its chunk log2-decays
    // (both directions) the reverse local state of the span, gathered as the
    // span is walked forwards: every token's input weighted by the decay of
    // the span's tokens before it; lb = log2 decay of the chunks walked
    constexpr int NBR = MODE == kModeStateBoth ? NB : 1;
    f32x4 Hr[NBR];
#pragma unroll
    for (int nb = 0; nb < NBR; ++nb) Hr[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    float lb = 0.f;
    auto state_ptr = [&](int64_t sp) -> T* {
        return (T*)p.states + (sp * p.H + h) * (int64_t)p.P * N;
    };
    // the same slot when span states are stored in float32 (plans 0 and 1)
    auto state_ptr_f = [&](int64_t sp) -> float* {
        return (float*)p.states + (sp * p.H + h) * (int64_t)p.P * N;
    };
    // (chunk_out) state slot of the span's first chunk: ceil(L / 64) slots
    // per sequence in batch mode, from the per-chunk table's offsets with
    // cu_seqlens
    const bool chunk_out = is_state(MODE) && p.chunk_out;
    const int64_t slot0 = !chunk_out ? 0
                          : p.nseq ? (int64_t)p.chunk_slot[vseq] + chunk0
                                   : (int64_t)seq_of * ((p.L + kChunk - 1) / kChunk) + chunk0;
    // fused kernel: one flag per work item, after the chains' header words
    uint32_t* const flags = p.sync + kSyncHeader + 2 * (int64_t)p.batch * ngrp * p.npg;

    // The fused kernel's fold of the earlier spans' published states into
    // the state entering the span, H <- a_j H + S_j in fp32 from the initial
    // state: the coherent loads go out up to U spans at a time (at most 128
    // registers of raw state), the first U with the first chunk's tiles.
    using R4 = typename Vec<T>::x4;
    constexpr int U = imin_c(kFuseSpans, 128 / (NB * (int)sizeof(T)));
    float fa[U];
    R4 fst[U][NB];
    int64_t fold_at = span - kin;  // next span to fold
    auto fold_issue = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t sj = fold_at + u;
            if (sj >= span) break;  // the same for the whole wave
            const T* st = state_ptr(sj);
            fa[u] = __uint_as_float(coherent_load32((const uint32_t*)&p.decay[sj * p.H + h]));
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) fst[u][nb] = coherent_load_raw4(st + state_off(pb, nb, lane, NB));
        }
    };
    auto fold_apply = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (fold_at + u >= span) break;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) Hs[nb] = fa[u] * Hs[nb] + widen4(fst[u][nb]);
        }
        fold_at += U;
    };

    if constexpr (SCANL) {
        // mask fragment halves that stay zero: tiles above the diagonal
        // (tb, sb) = (0, 1) and (2, 3)
        for (int i = tid; i < HG * 2 * 64; i += Cf::TH) {
            const int hh = i / 128, k = (i / 64) & 1, l = i & 63;
            sm.lf[hh][k ? lslot(2, 1) : lslot(0, 0)][1][l] = X4{};
        }
    }

    // y row of token t of chunk c: yc0 + c * ycs + yoff[t / 16] for this lane's t
    T* const yc0 = (T*)p.y + pcol0 + w4 * 16 + 4 * g + (int64_t)h * p.ys_h + tb0 * p.ys_t;
    const int64_t ycs = (int64_t)dstep * p.ys_t;
    int64_t yoff[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) yoff[tb] = (int64_t)(dir * (16 * tb + l16)) * p.ys_t;

    // One pass over the span's chunks, as a software pipeline: the local
    // state (SCAN false) or y (SCAN true).  Step c:
    //   wait for chunk c's tiles; barrier; (every fourth step) each wave
    //   forms one of the next four chunks' decay factors, barrier, and loads
    //   d_raw of the four after; issue chunk c+1's X and B tiles into the
    //   free buffers; (scan) the inter-chunk term H^T C^T and the masked
    //   C B^T, barrier, issue chunk c+1's C tile, write y; advance the state.
    // Only loads into LDS are in flight across a step, and the explicit wait
    // at its top covers them; the compiler itself never waits for them (the
    // restrict qualifiers below tell it that the step's LDS reads and the
    // loads it issues touch different buffers).  A pass leaves no load in
    // flight.
    auto run = [&](auto scan_tag) __attribute__((always_inline)) {
        constexpr bool SCAN = decltype(scan_tag)::value;
        // a chunk's decay factors, and the state update weights among them
        auto form_dec = [&](auto& D, uint32_t raw, int cl) {
            if constexpr (!std::is_same_v<std::decay_t<decltype(D)>, Decay>)
                decay_factors<T>(D, raw, p.d_init, cl, lane, MODE == kModeStateGrad);
            else
                decay_factors<T>(D, raw, p.d_init, cl, lane);
        };
        auto state_w = [&](const auto& D, int s0) -> const float* {
            if constexpr (!std::is_same_v<std::decay_t<decltype(D)>, Decay>) return &D.w[s0];
            else return MODE == kModeStateGrad ? &D.fe[s0] : &D.w[s0];
        };
        if constexpr (MODE != kModeScan) {  // (span_scan issued these before its entering state)
            if (w4 < nck) issue_d(w4, sm.dr[0][w4][q]);
            if (kWaves + w4 < nck) issue_d(kWaves + w4, sm.dr[1][w4][q]);
            issue_xb(0, sm.xs[0][q], sm.bs[0]);
            if (SCAN) issue_c(0, sm.cs);
        }
        if (MODE == kModeFused && SCAN) {
            // the fused kernel's fold loads go out with the first tiles
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) Hs[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (active) {
                if (p.init) {
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) Hs[nb][i] = p.init[hseq + np_off(nb, i)];
                }
                if (kin > 0) fold_issue();
            }
        }
        vm_wait<0>();
        if (MODE == kModeFused && SCAN && active && kin > 0) {
            fold_apply();
            while (fold_at < span) {
                fold_issue();
                fold_apply();
            }
        }
        if (w4 < nck) form_dec(sm.dec[w4][q], sm.dr[0][w4][q][lane], clen_of(w4));

        for (int c = 0; c < nck; ++c) {
            const bool last = c + 1 == nck;
            const int buf = c & 1;
            const int cl = clen_of(c);
            const auto& D = sm.dec[c % kWaves][q];

            // After chunk c's loads this wave issued, in an active scan wave,
            // exactly four y stores (the previous chunk is full), else nothing.
            // (chunk_out) after chunk c's loads, an active state wave stored
            // exactly NB entries of the previous chunk's state (a carried
            // walk stores none at its first chunk).
            if (SCAN && active && c > 0) vm_wait<4>();
            else if (!SCAN && chunk_out && active && c > 0 && (c > 1 || !p.chunk_run)) vm_wait<NB>();
            else vm_wait<0>();
            block_sync();  // every wave's loads of chunk c are in LDS
            if (c > 0 && c % kWaves == 0) {
                // batch c/4: its d_raw was loaded four steps ago
                const int bb = (c / kWaves) & 1;
                if (c + w4 < nck)
                    form_dec(sm.dec[w4][q], sm.dr[bb][w4][q][lane], clen_of(c + w4));
                block_sync();
                if (c + kWaves + w4 < nck) issue_d(c + kWaves + w4, sm.dr[bb ^ 1][w4][q]);
            }

            auto body = [&](const T* __restrict__ xt, const T* __restrict__ bt_tile,
                            const T* __restrict__ ct, T* __restrict__ xn, T* __restrict__ bn,
                            T* __restrict__ cn) {
                if (!last) issue_xb(c + 1, xn, bn);
                if (!SCAN && chunk_out && p.chunk_run && active && c > 0) {
                    // (carried chunk states) the span-local state entering
                    // this chunk: the chunks walked before it (none before
                    // the first: its slot is not written, and not read)
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
                        store4_async(state_ptr(slot0 + ck(c)) + state_off(pb, nb, lane, NB), Hs[nb]);
                }

                if constexpr (SCAN) {
                    const auto& Ds = dep_on(scan_tag, D);  // the scan's full factor set
                    // C rows 16*tb + l16, the B operand of C B^T and H^T C^T
                    X8 cf[4][KN];
#pragma unroll
                    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
                        for (int kk = 0; kk < KN; ++kk) cf[tb][kk] = tile_frag<N>(ct, 16 * tb + l16, kk, g);
                    // inter-chunk term y^T = H^T C^T with the state entering chunk c
                    f32x4 ye[4];
                    {
                        X8 hf[KN];
#pragma unroll
                        for (int kk = 0; kk < KN; ++kk) {
                            X4 lo, hi = {};
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                lo[i] = cvt<T>(Hs[2 * kk][i]);
                                if (2 * kk + 1 < NB) hi[i] = cvt<T>(Hs[2 * kk + 1][i]);
                            }
                            hf[kk] = cat<X8, X4>(lo, hi);
                        }
#pragma unroll
                        for (int tb = 0; tb < 4; ++tb) {
                            ye[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                            for (int kk = 0; kk < KN; ++kk) ye[tb] = mma(hf[kk], cf[tb][kk], ye[tb]);
                        }
                    }
                    // C B^T tiles with t-block >= s-block, 3/3/2/2 per wave, masked
                    // with this quad's head decay
                    X8 a[KN];
                    auto bfrag = [&](int sb) {
#pragma unroll
                        for (int kk = 0; kk < KN; ++kk) a[kk] = tile_frag<N>(bt_tile, 16 * sb + l16, kk, g);
                    };
                    switch (w4) {
                        case 0:
                            bfrag(0);
                            mask_tile<0, 0>(sm, Ds, q, lane, a, cf[0]);
                            mask_tile<1, 0>(sm, Ds, q, lane, a, cf[1]);
                            mask_tile<2, 0>(sm, Ds, q, lane, a, cf[2]);
                            break;
                        case 1:
                            bfrag(1);
                            mask_tile<1, 1>(sm, Ds, q, lane, a, cf[1]);
                            mask_tile<2, 1>(sm, Ds, q, lane, a, cf[2]);
                            mask_tile<3, 1>(sm, Ds, q, lane, a, cf[3]);
                            break;
                        case 2:
                            bfrag(0);
                            mask_tile<3, 0>(sm, Ds, q, lane, a, cf[3]);
                            bfrag(2);
                            mask_tile<2, 2>(sm, Ds, q, lane, a, cf[2]);
                            break;
                        default:
                            bfrag(2);
                            mask_tile<3, 2>(sm, Ds, q, lane, a, cf[3]);
                            bfrag(3);
                            mask_tile<3, 3>(sm, Ds, q, lane, a, cf[3]);
                            break;
                    }
                    block_sync();  // masked fragments complete, C tile no longer read
                    if (!last) issue_c(c + 1, cn);

                    // X^T fragments in the K order of the mask tiles:
                    // tokens 32kk + 4g + (0..3) and 32kk + 16 + 4g + (0..3)
                    X8 xf[2];
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk)
                        xf[kk] = tok_frag(xt, 32 * kk + 4 * g, 32 * kk + 16 + 4 * g, w4, lane);
                    X8 lf[6];
#pragma unroll
                    for (int s = 0; s < 6; ++s) lf[s] = cat<X8, X4>(sm.lf[q][s][0][lane], sm.lf[q][s][1][lane]);
                    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int tb = 0; tb < 4; ++tb) {
                        // intra-chunk: y^T += X^T L^T (causal fragments only)
                        f32x4 yi = mma(xf[0], lf[lslot(tb, 0)], z);
                        if (tb >= 2) yi = mma(xf[1], lf[lslot(tb, 1)], yi);
                        const int t = 16 * tb + l16;
                        const float sc = Ds.fe[t];
                        f32x4 o;
#pragma unroll
                        for (int i = 0; i < 4; ++i) o[i] = yi[i] + sc * ye[tb][i];
                        if (active && t < cl) store4_async(yc0 + c * ycs + yoff[tb], o);
                    }
                }

                if (!(SCAN && last) || (SCAN && write_final)) {
                    // advance the state over this chunk: H = e^{cs_last} H + B^T (w X)
                    const float decay = chunk_decay(D);
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) Hs[nb] *= decay;
#pragma unroll
                    for (int kk = 0; kk < kChunk / 32; ++kk) {
                        const int s0 = 32 * kk + 8 * g;  // tokens s0 .. s0+7
                        f32x8 ws = ld8(state_w(D, s0));
                        if constexpr (MODE == kModeStateGrad) {
                            // e^{cs_s} does not vanish past a partial chunk's
                            // end (d_s does): rows there hold row 0 again
                            if (cl < kChunk) {
#pragma unroll
                                for (int j = 0; j < 8; ++j) ws[j] = s0 + j < cl ? ws[j] : 0.f;
                            }
                        }
                        const X8 xv = tok_frag(xt, s0, s0 + 4, w4, lane);
                        X8 b, bt[NB];
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb) bt[nb] = tok_frag(bt_tile, s0, s0 + 4, nb, lane);
#pragma unroll
                        for (int j = 0; j < 8; ++j) b[j] = cvt<T>((float)xv[j] * ws[j]);
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb) Hs[nb] = mma(bt[nb], b, Hs[nb]);
                        if constexpr (MODE == kModeStateBoth) {
                            const float pre = fexp2(lb);  // the chunks before this one
                            const f32x8 wr = ld8(&D.wr[s0]);
#pragma unroll
                            for (int j = 0; j < 8; ++j) b[j] = cvt<T>((float)xv[j] * (wr[j] * pre));
#pragma unroll
                            for (int nb = 0; nb < NB; ++nb) Hr[nb] = mma(bt[nb], b, Hr[nb]);
                        }
                    }
                }
                if (!SCAN && w4 == 0) logdec2 += D.cs2[kChunk - 1];
                if (MODE == kModeStateBoth) lb += D.cs2[kChunk - 1];
                if (!SCAN && chunk_out && !p.chunk_run) {
                    // this chunk's local state; the next starts from zero
                    if (active) {
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb)
                            store4_async(state_ptr(slot0 + c) + state_off(pb, nb, lane, NB), Hs[nb]);
                    }
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) Hs[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            };
            body(sm.xs[buf][q], sm.bs[buf], sm.cs, sm.xs[buf ^ 1][q], sm.bs[buf ^ 1], sm.cs);
        }
    };

    if constexpr (is_state(MODE)) {
        run(std::false_type{});
        if (chunk_out && !p.chunk_run) {
            // chunk w4's decay (its factors are still in slot w4: K <= 4)
            if (pg == 0 && w4 < nck && live && lane == 0)
                p.decay[(slot0 + w4) * p.H + h] = fexp2(sm.dec[w4][q].cs2[kChunk - 1]);
            return;
        }
        if (chunk_out) {
            // (carried chunk states) walk step w4's decay slot: the decay
            // product of the steps before it (their factors are still in
            // slots 0..3: K <= 4); the span's whole local state and decay
            if (pg == 0 && w4 < nck && live && lane == 0) {
                float l2 = 0.f;
                for (int j = 0; j < w4; ++j) l2 += sm.dec[j][q].cs2[kChunk - 1];
                p.decay[(slot0 + ck(w4)) * p.H + h] = fexp2(l2);
            }
            if (active) {
                T* const sp = (T*)p.span_states + (span * p.H + h) * (int64_t)p.P * N;
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) store4(sp + state_off(pb, nb, lane, NB), Hs[nb]);
            }
            if (pg == 0 && w4 == 0 && live && lane == 0) p.span_decay[span * p.H + h] = fexp2(logdec2);
            return;
        }
        if (active) {
            if (p.state_f32) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) store4(state_ptr_f(span) + state_off(pb, nb, lane, NB), Hs[nb]);
            } else {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) store4(state_ptr(span) + state_off(pb, nb, lane, NB), Hs[nb]);
            }
        }
        if (pg == 0 && w4 == 0 && live && lane == 0) p.decay[span * p.H + h] = fexp2(logdec2);
        if constexpr (MODE == kModeStateBoth) {
            // the reverse pass's span kin' = sps - 1 - kin of the sequence
            // covers the same tokens (whole spans: L a multiple of 64 K)
            const int64_t rspan = span + (p.sps - 1 - 2 * (int64_t)kin);
            if (active) {
                if (p.state_f32) {
                    float* const rp = (float*)p.rev_states + (rspan * p.H + h) * (int64_t)p.P * N;
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) store4(rp + state_off(pb, nb, lane, NB), Hr[nb]);
                } else {
                    T* const rp = (T*)p.rev_states + (rspan * p.H + h) * (int64_t)p.P * N;
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) store4(rp + state_off(pb, nb, lane, NB), Hr[nb]);
                }
            }
            if (pg == 0 && w4 == 0 && live && lane == 0) p.rev_decay[rspan * p.H + h] = fexp2(logdec2);
        }
        return;
    }

    if constexpr (MODE == kModeFused) {
        if (kin + 1 < p.sps) {
            // the span's local state and decay, published for the later spans
            run(std::false_type{});
            if (active) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    coherent_store4(state_ptr(span) + state_off(pb, nb, lane, NB), Hs[nb]);
            }
            if (w4 == 0 && live && lane == 0)
                coherent_store32((uint32_t*)&p.decay[span * p.H + h], __float_as_uint(fexp2(logdec2)));
            drain_vm();    // this wave's stores have reached the point of coherence
            block_sync();  // so have every wave's; the pass's LDS is free again
            if (tid == 0) coherent_store32(flags + logical, epoch);
        }
        if (kin > 0) {
            // Wait for the flags of spans 0 .. kin-1 of this sequence (same
            // head group and column group), lane j of wave 0 polling span j.
            // The wait is bounded: flags that never come (a header not
            // zero-filled before first use) are counted in the header and
            // the fold goes on without them.
            if (wave == 0) {
                const uint32_t* f = flags + ((span - kin + (lane < kin ? lane : 0)) * ngrp + hgi) * p.npg + pg;
                uint32_t budget = kSpinBudget;
                while (!__all(lane >= kin || coherent_load32(f) == epoch)) {
                    if (--budget == 0) {
                        if (lane == 0)
                            __hip_atomic_fetch_add(p.sync + kSyncTimeouts, 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
            }
            block_sync();
        }
    }

    if constexpr (MODE == kModeScan) {
        // The first chunk's tiles and d_raw go out first: their loads into
        // LDS overlap the forming of the entering state below.
        if (w4 < nck) issue_d(w4, sm.dr[0][w4][q]);
        if (kWaves + w4 < nck) issue_d(kWaves + w4, sm.dr[1][w4][q]);
        issue_xb(0, sm.xs[0][q], sm.bs[0]);
        issue_c(0, sm.cs);
        // (span_scan) the state entering the span: as state_pass left it in
        // place of the span state, or folded here span by span
        if (active) {
            if (!folds) {
                if (p.state_f32) {
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) Hs[nb] = load4(state_ptr_f(span) + state_off(pb, nb, lane, NB));
                } else {
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) Hs[nb] = load4(state_ptr(span) + state_off(pb, nb, lane, NB));
                }
            } else {
                if (p.init) {
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) Hs[nb][i] = p.init[hseq + np_off(nb, i)];
                }
                for (int64_t sj = span - kin; sj < span; ++sj) {
                    const float a = p.decay[sj * p.H + h];
                    if (p.state_f32) {
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb)
                            Hs[nb] = a * Hs[nb] + load4(state_ptr_f(sj) + state_off(pb, nb, lane, NB));
                    } else {
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb)
                            Hs[nb] = a * Hs[nb] + load4(state_ptr(sj) + state_off(pb, nb, lane, NB));
                    }
                }
            }
        }
    }

    if constexpr (SCANL) {
        run(std::true_type{});
        if (write_final && active) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int i = 0; i < 4; ++i) p.final_state[hseq + np_off(nb, i)] = Hs[nb][i];
        }
    }
}

template <typename T, int N, int HG, int MODE>
__global__ __launch_bounds__(kThreads * HG, (span_occupancy<T, N, HG, MODE>())) void span_kernel(
    KParams p) {
    __shared__ Smem<T, N, HG, !is_state(MODE), MODE == kModeStateBoth> sm;
    touch_args(p);
    span_body<T, N, HG, MODE>(p, blockIdx.x, sm);
}

// The backward pass's two chunk-state passes in one launch (they are
// independent): workgroups below na form the states of the forward
// direction from (B, x), the rest the output-gradient states from (C, dy).
// na is a multiple of the XCD count, so each half keeps its XCD-aware order.
template <typename T, int N>
__global__ __launch_bounds__(kThreads, (span_occupancy<T, N, 1, kModeState>())) void span_state_pair_kernel(
    KParams pa, KParams pb, int64_t na) {
    __shared__ Smem<T, N, 1, false> sm;
    if ((int64_t)blockIdx.x < na) {
        touch_args(pa);
        span_body<T, N, 1, kModeState>(pa, blockIdx.x, sm);
    } else {
        touch_args(pb);
        span_body<T, N, 1, kModeStateGrad>(pb, blockIdx.x - na, sm);
    }
}

// A 16-byte store the compiler's wait counting does not see (the s_nop
// covers the hazard of a VALU write to the data registers right after a
// store of more than 8 bytes).
template <typename V16>
__device__ __forceinline__ void store16_async(V16* p, const V16& v) {
    static_assert(sizeof(V16) == 16, "16-byte vector");
    typedef uint32_t U4 __attribute__((ext_vector_type(4)));
    const U4 w = __builtin_bit_cast(U4, v);
    asm volatile("global_store_dwordx4 %0, %1, off\n\ts_nop 0" ::"v"(p), "v"(w) : "memory");
}

// Walk the spans of one sequence for V = 16 bytes of consecutive stored
// state entries: replace each span state S_k (input type) by the state
// entering the span and carry H <- decay_k H + S_k in fp32; H after the last
// span is the final state.  Stored entry o of a (span, head) block holds
// state (n, p) as laid out by state_off(); init/final are [N][P].
template <typename TS>
__device__ __forceinline__ void state_pass_body(const KParams& p, int64_t gid) {
    // spans per batch.  Two batches of loads (two each per span) and one
    // batch of stores can be in flight, 5U vector-memory operations, and
    // the hardware counts at most 63: U = 8 keeps the waits exact.
    constexpr int U = 8;
    constexpr int V = 16 / sizeof(TS);   // state entries per thread
    typedef TS TSV __attribute__((ext_vector_type(V)));
    typedef float FV __attribute__((ext_vector_type(V)));
    const int N = p.N, NB = p.N / 16;
    const int EV = p.P * N / V;
    const int64_t S = p.nseq ? p.nseq : p.batch;
    if (gid >= S * p.H * EV) return;
    // (divisions as multiply-highs set by the launcher: threads < 2^31)
    const uint32_t g32 = (uint32_t)gid, r1 = fdiv(g32, p.dc.by_ev);
    const int ev = (int)(g32 - r1 * (uint32_t)EV);
    const uint32_t i32 = fdiv(r1, p.dc.by_h);
    const int h = (int)(r1 - i32 * (uint32_t)p.H);
    const int64_t i = i32;
    int64_t s0, s1;
    if (p.nseq) {
        s0 = p.span_off[i];
        s1 = p.span_off[i + 1];
    } else {
        s0 = i * p.sps;
        s1 = s0 + p.sps;
    }
    int idx[V];  // [N][P] position of each entry
#pragma unroll
    for (int j = 0; j < V; ++j) {
        const int o = ev * V + j;
        const int lane = (o >> 2) & 63, q = o >> 8;
        const int qb = (int)fdiv((uint32_t)q, p.dc.by_nb);  // q / NB
        const int n = 16 * (q - qb * NB) + 4 * (lane >> 4) + (o & 3);
        const int pp = 16 * qb + (lane & 15);
        idx[j] = n * p.P + pp;
    }
    const int64_t hb = (i * p.H + h) * (int64_t)N * p.P;
    FV run = {};
    if (p.init) {
#pragma unroll
        for (int j = 0; j < V; ++j) run[j] = p.init[hb + idx[j]];
    }
    TSV* st = (TSV*)p.states;
    // span number k of the walk: s0 + k, or s1 - 1 - k walking backwards
    const int64_t ns = s1 - s0;
    auto span_at = [&](int64_t k) { return p.pass_desc ? s1 - 1 - k : s0 + k; };
    // Two batches of U spans in flight: batch k + U is loaded while batch k
    // is combined, so a long walk pays about one memory latency per batch
    // of U spans rather than one per batch plus the combine.  The loads are
    // branch-free (positions past the walk re-read its last span, unused)
    // and the stores are issued by store16_async, which the compiler's wait
    // counting does not see: so the only waits it places are the exact ones
    // for the batch being combined.  Loads and stores retire in order, so a
    // wait that counts only loads still covers every load it names.
    TSV va[U], vb[U];
    float da[U], db[U];
    auto load = [&](int64_t k, TSV (&v)[U], float (&d)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t sp = span_at(k + u < ns ? k + u : ns - 1);
            v[u] = st[(sp * p.H + h) * EV + ev];
            d[u] = p.decay[sp * p.H + h];
        }
    };
    auto combine = [&](int64_t k, const TSV (&v)[U], const float (&d)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            TSV o;
#pragma unroll
            for (int j = 0; j < V; ++j) o[j] = (TS)run[j];
            const bool in = k + u < ns;  // positions past the walk change nothing
            if (in) store16_async(&st[(span_at(k + u) * p.H + h) * EV + ev], o);
#pragma unroll
            for (int j = 0; j < V; ++j) run[j] = in ? d[u] * run[j] + (float)v[u][j] : run[j];
        }
    };
    if (ns > 0) {
        load(0, va, da);
        for (int64_t k = 0; k < ns; k += 2 * U) {
            load(k + U, vb, db);
            combine(k, va, da);
            if (k + U >= ns) break;
            load(k + 2 * U, va, da);
            combine(k + U, vb, db);
        }
    }
    if (p.final_state) {
#pragma unroll
        for (int j = 0; j < V; ++j) p.final_state[hb + idx[j]] = run[j];
    }
}

template <typename TS>
__global__ __launch_bounds__(256) void state_pass_kernel(KParams p) {
    touch_args(p);
    state_pass_body<TS>(p, (int64_t)blockIdx.x * 256 + threadIdx.x);
}

// Two independent state passes in one launch: workgroups below na walk pa's
// spans, the rest pb's.
template <typename TS>
__global__ __launch_bounds__(256) void state_pass_pair_kernel(KParams pa, KParams pb, int64_t na) {
    if ((int64_t)blockIdx.x < na) {
        touch_args(pa);
        state_pass_body<TS>(pa, (int64_t)blockIdx.x * 256 + threadIdx.x);
    } else {
        touch_args(pb);
        state_pass_body<TS>(pb, ((int64_t)blockIdx.x - na) * 256 + threadIdx.x);
    }
}

// Zero words [0, nwords) of the workspace header and the fused launch's
// chain words and flags (a fill kernel rather than a memset, so the call
// can be captured in a graph).
__global__ __launch_bounds__(256) void fused_reset_kernel(uint32_t* sync, int64_t nwords) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < nwords) sync[i] = 0u;
}

// One workgroup: sanitize cu_seqlens (clamped running maximum, first entry
// 0), count each sequence's spans, prefix-sum them and write the span table.
// Tail slots up to nspan are marked empty (seq = -1).
constexpr int kTab = 1024;
__global__ __launch_bounds__(kTab) void span_table_kernel(const int32_t* cu, int32_t nseq,
                                                          int64_t T, int32_t K, int64_t nspan,
                                                          int32_t* cu_san, int32_t* span_off,
                                                          int4* table) {
    __shared__ int32_t smax[kTab];
    __shared__ int32_t ssum[kTab];
    const int tid = threadIdx.x;
    int32_t carry_max = 0;   // sanitized cu of the last sequence end so far
    int32_t carry_off = 0;   // spans so far
    if (tid == 0) cu_san[0] = 0;
    for (int32_t base = 0; base < nseq; base += kTab) {
        const int32_t i = base + tid;  // sequence index
        int32_t e = 0;
        if (i < nseq) {
            int64_t v = cu[i + 1];
            v = v < 0 ? 0 : (v > T ? T : v);
            e = (int32_t)v;
        }
        smax[tid] = e;
        __syncthreads();
        for (int off = 1; off < kTab; off <<= 1) {
            const int32_t o = tid >= off ? smax[tid - off] : 0;
            __syncthreads();
            smax[tid] = max(smax[tid], o);
            __syncthreads();
        }
        const int32_t end = max(carry_max, smax[tid]);
        const int32_t beg = tid == 0 ? carry_max : max(carry_max, smax[tid - 1]);
        const int64_t len = i < nseq ? (int64_t)end - beg : 0;
        const int64_t nch = (len + kChunk - 1) / kChunk;
        const int32_t nsp = (int32_t)((nch + K - 1) / K);
        ssum[tid] = nsp;
        __syncthreads();
        for (int off = 1; off < kTab; off <<= 1) {
            const int32_t o = tid >= off ? ssum[tid - off] : 0;
            __syncthreads();
            ssum[tid] += o;
            __syncthreads();
        }
        const int32_t off0 = carry_off + ssum[tid] - nsp;
        if (i < nseq) {
            cu_san[i + 1] = end;
            span_off[i] = off0;
            for (int32_t k = 0; k < nsp && off0 + k < nspan; ++k) {
                const int32_t c0 = k * K;
                const int32_t nc = (int32_t)imin(K, nch - c0);
                table[off0 + k] = make_int4(i, c0, nc, 0);
            }
        }
        const int32_t tile_max = smax[kTab - 1];
        const int32_t tile_sum = ssum[kTab - 1];
        __syncthreads();
        carry_max = max(carry_max, tile_max);
        carry_off += tile_sum;
    }
    if (tid == 0) span_off[nseq] = carry_off;
    for (int64_t k = (int64_t)carry_off + tid; k < nspan; k += kTab) table[k] = make_int4(-1, 0, 0, 0);
}

template <typename T, int N, int HG, int MODE>
hipError_t launch_span_hg(const KParams& p, int hg, hipStream_t s) {
    const int64_t nreal = p.nspan * ((p.H + hg - 1) / hg) * p.npg;
    if (nreal == 0) return hipSuccess;
    // the fused kernel takes one ticket per workgroup: exactly nreal of them
    const int64_t grid = MODE == kModeFused ? nreal : (nreal + kXcds - 1) / kXcds * kXcds;
    KParams q = p;
    set_decode(q, hg);
    hipLaunchKernelGGL((span_kernel<T, N, HG, MODE>), dim3((unsigned)grid), dim3(kThreads * HG), 0,
                       s, q);
    return hipGetLastError();
}

// Instantiated for 1 and 2 heads per workgroup, up to the most the kernel
// can carry at this d_state.
template <typename T, int N, int MODE>
hipError_t launch_span_t(const KParams& p, hipStream_t s) {
    constexpr int MAXH = !is_state(MODE) ? heads_scan(N, sizeof(T)) : heads_state(N, sizeof(T));
    const int hg = !is_state(MODE) ? p.hg_scan : p.hg_state;
    if (hg == 1) return launch_span_hg<T, N, 1, MODE>(p, 1, s);
    if (hg == 2 && MAXH >= 2) return launch_span_hg<T, N, (MAXH >= 2 ? 2 : 1), MODE>(p, 2, s);
    return hipErrorInvalidValue;
}

template <int MODE>
hipError_t launch_span(const KParams& p, int dtype, int N, hipStream_t s) {
    if (dtype == 1) {
        switch (N) {
            case 16: return launch_span_t<bf16, 16, MODE>(p, s);
            case 32: return launch_span_t<bf16, 32, MODE>(p, s);
            case 64: return launch_span_t<bf16, 64, MODE>(p, s);
            case 128: return launch_span_t<bf16, 128, MODE>(p, s);
            case 256: return launch_span_t<bf16, 256, MODE>(p, s);
        }
    } else {
        switch (N) {
            case 16: return launch_span_t<float, 16, MODE>(p, s);
            case 32: return launch_span_t<float, 32, MODE>(p, s);
            case 64: return launch_span_t<float, 64, MODE>(p, s);
            case 128: return launch_span_t<float, 128, MODE>(p, s);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace

int span_max_heads(int dtype, int N, bool scan) {
    const int esz = dtype == 1 ? 2 : 4;
    return scan ? heads_scan(N, esz) : heads_state(N, esz);
}

size_t span_lds_bytes(int dtype, int N, bool scan) {
#define SSD_LDS(T, NN)                                                 \
    (scan ? sizeof(Smem<T, NN, heads_scan(NN, sizeof(T)), true>)       \
          : sizeof(Smem<T, NN, heads_state(NN, sizeof(T)), false>))
    if (dtype == 1) {
        switch (N) {
            case 16: return SSD_LDS(bf16, 16);
            case 32: return SSD_LDS(bf16, 32);
            case 64: return SSD_LDS(bf16, 64);
            case 128: return SSD_LDS(bf16, 128);
            case 256: return SSD_LDS(bf16, 256);
        }
    } else if (dtype == 0) {
        switch (N) {
            case 16: return SSD_LDS(float, 16);
            case 32: return SSD_LDS(float, 32);
            case 64: return SSD_LDS(float, 64);
            case 128: return SSD_LDS(float, 128);
        }
    }
#undef SSD_LDS
    return 0;
}

hipError_t launch_span_table(const int32_t* cu_raw, int32_t nseq, int64_t T, int32_t K,
                             int64_t nspan, int32_t* cu_san, int32_t* span_off, int4* table,
                             hipStream_t s) {
    hipLaunchKernelGGL(span_table_kernel, dim3(1), dim3(kTab), 0, s, cu_raw, nseq, T, K, nspan,
                       cu_san, span_off, table);
    return hipGetLastError();
}

hipError_t launch_fused_reset(uint32_t* sync, int64_t nwords, hipStream_t s) {
    if (nwords <= 0) return hipSuccess;
    hipLaunchKernelGGL(fused_reset_kernel, dim3((unsigned)((nwords + 255) / 256)), dim3(256), 0, s,
                       sync, nwords);
    return hipGetLastError();
}

hipError_t launch_span_state(const KParams& p, int dtype, int N, hipStream_t s) {
    return p.wmode ? launch_span<kModeStateGrad>(p, dtype, N, s) : launch_span<kModeState>(p, dtype, N, s);
}

hipError_t launch_span_scan(const KParams& p, int dtype, int N, hipStream_t s) {
    return p.fuse_pass == 2 ? launch_span<kModeFused>(p, dtype, N, s)
                            : launch_span<kModeScan>(p, dtype, N, s);
}

// Both directions' span states in one walk (one head per workgroup; batch
// mode, whole spans).
hipError_t launch_span_state_both(const KParams& p, int dtype, int N, hipStream_t s) {
    if ((p.hg_state != 1 && !(p.hg_state == 2 && dtype == 1)) || p.nseq) return hipErrorInvalidValue;
    if (dtype == 1 && p.hg_state == 2) {
        switch (N) {
            case 16: return launch_span_hg<bf16, 16, 2, kModeStateBoth>(p, 2, s);
            case 32: return launch_span_hg<bf16, 32, 2, kModeStateBoth>(p, 2, s);
            case 64: return launch_span_hg<bf16, 64, 2, kModeStateBoth>(p, 2, s);
            case 128: return launch_span_hg<bf16, 128, 2, kModeStateBoth>(p, 2, s);
        }
    } else if (dtype == 1) {
        switch (N) {
            case 16: return launch_span_hg<bf16, 16, 1, kModeStateBoth>(p, 1, s);
            case 32: return launch_span_hg<bf16, 32, 1, kModeStateBoth>(p, 1, s);
            case 64: return launch_span_hg<bf16, 64, 1, kModeStateBoth>(p, 1, s);
            case 128: return launch_span_hg<bf16, 128, 1, kModeStateBoth>(p, 1, s);
        }
    } else {
        switch (N) {
            case 16: return launch_span_hg<float, 16, 1, kModeStateBoth>(p, 1, s);
            case 32: return launch_span_hg<float, 32, 1, kModeStateBoth>(p, 1, s);
            case 64: return launch_span_hg<float, 64, 1, kModeStateBoth>(p, 1, s);
            case 128: return launch_span_hg<float, 128, 1, kModeStateBoth>(p, 1, s);
        }
    }
    return hipErrorInvalidValue;
}
hipError_t launch_span_state_pair(const KParams& pa, const KParams& pb, int dtype, int N,
                                  hipStream_t s) {
    const int64_t n = pa.nspan * pa.H * pa.npg;  // one head per workgroup (both halves)
    if (n == 0) return hipSuccess;
    const int64_t na = (n + kXcds - 1) / kXcds * kXcds;
    KParams qa = pa, qb = pb;
    set_decode(qa, 1);
    set_decode(qb, 1);
#define SSD_PAIR(T, NN) \
    hipLaunchKernelGGL((span_state_pair_kernel<T, NN>), dim3((unsigned)(2 * na)), dim3(kThreads), 0, s, qa, qb, na)
    if (dtype == 1) {
        switch (N) {
            case 16: SSD_PAIR(bf16, 16); break;
            case 32: SSD_PAIR(bf16, 32); break;
            case 64: SSD_PAIR(bf16, 64); break;
            case 128: SSD_PAIR(bf16, 128); break;
            default: return hipErrorInvalidValue;
        }
    } else {
        switch (N) {
            case 16: SSD_PAIR(float, 16); break;
            case 32: SSD_PAIR(float, 32); break;
            case 64: SSD_PAIR(float, 64); break;
            case 128: SSD_PAIR(float, 128); break;
            default: return hipErrorInvalidValue;
        }
    }
#undef SSD_PAIR
    return hipGetLastError();
}

hipError_t launch_state_pass_pair(const KParams& pa, const KParams& pb, int dtype, hipStream_t s) {
    const int64_t S = pa.nseq ? pa.nseq : pa.batch;
    const int V = dtype == 1 ? 8 : 4;
    const int64_t n = S * pa.H * (int64_t)pa.P * pa.N / V;
    if (n == 0) return hipSuccess;
    const int64_t na = (n + 255) / 256;
    KParams qa = pa, qb = pb;
    set_pass_decode(qa, V);
    set_pass_decode(qb, V);
    if (dtype == 1)
        hipLaunchKernelGGL(state_pass_pair_kernel<bf16>, dim3((unsigned)(2 * na)), dim3(256), 0, s, qa, qb, na);
    else
        hipLaunchKernelGGL(state_pass_pair_kernel<float>, dim3((unsigned)(2 * na)), dim3(256), 0, s, qa, qb, na);
    return hipGetLastError();
}

hipError_t launch_state_pass(const KParams& p, int dtype, hipStream_t s) {
    const int64_t S = p.nseq ? p.nseq : p.batch;
    const bool s16 = dtype == 1 && !p.state_f32;  // span states stored in bf16
    const int V = s16 ? 8 : 4;
    const int64_t n = S * p.H * (int64_t)p.P * p.N / V;
    if (n == 0) return hipSuccess;
    const dim3 grid((unsigned)((n + 255) / 256));
    KParams q = p;
    set_pass_decode(q, V);
    if (s16)
        hipLaunchKernelGGL(state_pass_kernel<bf16>, grid, dim3(256), 0, s, q);
    else
        hipLaunchKernelGGL(state_pass_kernel<float>, grid, dim3(256), 0, s, q);
    return hipGetLastError();
}

}  // namespace ssd
