// Head-wave span kernels for bf16 inputs on gfx950 (MI355X).
//
// Same scan, same chunked form and same span decomposition as the span
// kernels of ssd_kernels.hip ("长序列 Mamba 多卡训练，算力和显存怎么同时省", §一:
// a dense diagonal block per 64-token chunk plus a state handed across chunk
// borders; "Mamba-2架构与LaCT并行计算技术解析", §1.1 for the recurrence), with a
// different split of a chunk's work over the waves of a workgroup:
//
//   WPH = 4 / NPB waves carry one head, each holding the state of 16*NPB
//   headdim columns (NPB = 4: all 64 columns of a column group in one wave;
//   NPB = 2: two waves of 32 columns), and each does every product of its
//   head and columns itself: C Hprev, the intra-chunk product and the state
//   update.  The HG heads of a workgroup share one B / C group, its LDS
//   tiles and one causal C B^T per chunk, formed by all its waves together.
//
// Rescaled state.  Each wave keeps S = 2^{-la} H, with la (<= 0, >= -64) a
// running log2 decay of its head.  With cs the within-chunk cumulative log2
// decay (cs_last at the chunk's end) and the scaled inputs
//   Xs_s = 2^{-cs_s - la} d_s X_s      (at most 2^64 times d_s X_s),
// a chunk is
//   y_t = 2^{cs_t + la} ( C_t S + sum_{s <= t} (C_t . B_s) Xs_s )
//   S'  = S + sum_s B_s^T Xs_s,        la' = la + cs_last,
// so the per-head decay enters only through the row scales of Xs and y:
// C B^T needs just the causal mask and is the same for every head of the
// group, and no decay multiplies the state element by element.  When
// la + cs_last would fall below -64 the chunk first folds 2^{la} into S and
// restarts la at 0; only a chunk whose own decay exceeds 2^{-64} (then
// factors like 2^{-cs_s} could overflow) takes the explicit form:
//   y_t = 2^{cs_t} C_t S + sum_{s <= t} (C_t . B_s) 2^{cs_t - cs_s} d_s X_s,
//   S' = 2^{cs_last} S + sum_s B_s^T 2^{cs_last - cs_s} d_s X_s,  la' = 0,
// with the decay mask applied to each head's C B^T before the exponential.
//
// Tiles are double-buffered and loaded straight from global memory into LDS
// one chunk ahead (global_load_lds_dwordx4) in the column-blocked layout of
// ssd_device.h; d_raw runs two chunks ahead, and every wave of a head forms
// the head's next decay factors while the current chunk is computed.
//
// Modes: kHwState writes each span's local state (from a zero state) and
// its decay product; kHwScan starts from the state entering the span, as
// the state pass left it in the span's slot, and writes y.  The state pass
// between them is state_pass_kernel of ssd_kernels.hip (same state layout).
#include "ssd_device.h"

namespace ssd {
namespace {

enum { kHwState = 0, kHwScan = 1 };

// log2 of the largest factor the rescaled state and inputs may carry
constexpr float kRescaleLog2 = 64.f;

template <int N, int HG, int NPB>
struct HwCfg {
    static constexpr int WPH = 4 / NPB;              // waves per head (64 columns)
    static constexpr int NW = HG * WPH;              // waves per workgroup
    static constexpr int TH = 64 * NW;               // threads per workgroup
    static constexpr int NB = N / 16;                // 16-row blocks of the state
    static constexpr int KN = N / 32;                // K = 32 steps over d_state
    static constexpr int XI = 8;                     // 1 KB loads per 64 x 64 X tile
    static constexpr int XIW = XI / WPH;             // ... per wave of its head
    static constexpr int BI = N / 8;                 // 1 KB loads per 64 x N B / C tile
    static constexpr int BIW = (BI + NW - 1) / NW;   // ... per wave (most)
    static_assert(N % 32 == 0 && (NPB == 2 || NPB == 4), "head-wave shape");
};

// One head's factors for one chunk (cs = within-chunk cumulative log2
// decay, c_k = cs at the end of 16-token block k-1, c_0 = 0; la the head's
// running log2 scale, after any restart at this chunk's start):
//   fe = 2^{cs_t + la}       output row scale
//   w                        Xs weights: 2^{-cs_s - la} d_s, or in the
//                            explicit form 2^{cs_last - cs_s} d_s
//   cs2, dt, fa, fb, fm      explicit form's mask: 2^{cs_t - cs_s} d_s is
//                            computed directly on the diagonal 16x16 tiles
//                            and as fa_s fm(tb,sb) fb_t off them
//   hpre                     1, or 2^{la before} when la restarts here
//   hpost                    1, or 2^{cs_last} (explicit form)
//   slow                     1 for the explicit form
//   la, lsum                 la after the chunk; the sum of chunk log2 decays
struct __attribute__((aligned(16))) HwDecay {
    float fe[kChunk];
    float w[kChunk];
    float cs2[kChunk];
    float dt[kChunk];
    float fa[kChunk];
    float fb[kChunk];
    float fm[kChunk];   // lanes 0-5 meaningful
    float hpre, hpost, slow, la, lsum, pad[3];
};

template <int N, int HG, int NPB, bool SCAN>
struct __attribute__((aligned(16))) HwSmem {
    bf16 xs[2][HG][kChunk * kPGroup];        // X of each head, this column group
    bf16 bs[2][kChunk * N];                  // B
    bf16 cs[SCAN ? 2 : 1][SCAN ? kChunk * N : 8];  // C (scan)
    // causal C B^T of the chunk, shared by the heads, as MFMA fragments:
    // slot (t-block, K half) -> tb0: 0, tb1: 1, tb2: 2+kk, tb3: 4+kk; half =
    // s-block & 1; lane l holds rows s = 16sb + 4(l/16) + i, column l%16
    bf16x4 cb[SCAN ? 6 : 1][2][SCAN ? 64 : 1];
    HwDecay dec[2][HG];                      // chunk parity, head
    __attribute__((aligned(16))) uint32_t dr[2][HG][kChunk];  // d_raw, chunk parity
};

template <int V> using ic = std::integral_constant<int, V>;

__device__ __forceinline__ constexpr int hw_lslot(int tb, int kk) {
    return tb == 0 ? 0 : (tb == 1 ? 1 : (tb == 2 ? 2 + kk : 4 + kk));
}
// the 10 causal 16x16 tiles (t-block, s-block) in a fixed order
constexpr int kTileTb[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
constexpr int kTileSb[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};

// Four bf16 outputs of one lane at sbase + voff bytes, for the lanes where
// pred holds.  The predicate goes into EXEC inside one asm statement, so the
// store needs no branch (a branch would end the compiler's scheduling
// region); the compiler does not count the store in its own waits (the
// kernel waits for it explicitly).  s_and_b64 writes SCC, so SCC is declared
// clobbered: the compiler must not keep a carry or a compare result in it
// across the statement (a 64-bit scalar pointer add split around it would
// otherwise take a wrong carry).
__device__ __forceinline__ void store4_masked(const bf16* sbase, uint32_t voff, const f32x4& v,
                                              bool pred) {
    bf16x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = (bf16)v[i];
    const uint64_t m = __ballot(pred);
    uint64_t save;
    asm volatile(
        "s_mov_b64 %0, exec\n\t"
        "s_and_b64 exec, exec, %1\n\t"
        "s_nop 0\n\t"
        "global_store_dwordx2 %2, %3, %4\n\t"
        "s_mov_b64 exec, %0"
        : "=&s"(save)
        : "s"(m), "v"(voff), "v"(o), "s"(sbase)
        : "memory", "scc");
}

// The head's decay factors for one chunk from d_raw as loaded into LDS (a
// bf16 value in the low half of its 32-bit slot).  Every wave of the head
// forms them (the same values, into the same slots) with no branch, so the
// compiler can interleave this short serial chain with the wave's MFMA work.
// la and lsum are the head's running values before the chunk, advanced in
// place; every lane computes them (wave-uniform), so no wave reads back what
// another of its lanes wrote -- the LDS copies are read after a barrier.
__device__ __forceinline__ void hw_decay(HwDecay& D, uint32_t raw, float d_init, int clen, int lane,
                                         float& la, float& lsum) {
    const float draw = __uint_as_float(raw << 16);
    const float dt = lane < clen ? softplus(draw + d_init) : 0.f;
    const float v = wave_prefix_sum(-dt * kLog2e);
    const float c1 = lane_value(v, 15), c2 = lane_value(v, 31);
    const float c3 = lane_value(v, 47), c4 = lane_value(v, 63);
    const int sb = lane >> 4;
    const float cbeg = sb == 0 ? 0.f : (sb == 1 ? c1 : (sb == 2 ? c2 : c3));
    const float cend = sb == 0 ? c1 : (sb == 1 ? c2 : (sb == 2 ? c3 : c4));
    // wave-uniform path choice
    const bool restart = la + c4 < -kRescaleLog2;
    const bool slow = c4 < -kRescaleLog2;
    const float lu = restart ? 0.f : la;  // la in use for this chunk
    D.fe[lane] = fexp2(v + lu);
    D.w[lane] = fexp2(slow ? c4 - v : -v - lu) * dt;
    D.cs2[lane] = v;
    D.dt[lane] = dt;
    D.fa[lane] = fexp2(cend - v) * dt;
    D.fb[lane] = fexp2(v - cbeg);
    {
        // lanes 0-5: (tb, sb) = (1,0) (2,0) (2,1) (3,0) (3,1) (3,2), 2^{c_tb - c_{sb+1}}
        const float ct = lane == 0 ? c1 : (lane < 3 ? c2 : c3);
        const float cs = (lane == 0 || lane == 1 || lane == 3) ? c1 : ((lane == 2 || lane == 4) ? c2 : c3);
        D.fm[lane] = fexp2(ct - cs);
    }
    const float la_next = slow ? 0.f : lu + c4, lsum_next = lsum + c4;
    // every lane stores the same wave-uniform values
    D.hpre = restart ? fexp2(la) : 1.f;
    D.hpost = slow ? fexp2(c4) : 1.f;
    D.slow = slow ? 1.f : 0.f;
    D.la = la_next;
    D.lsum = lsum_next;
    la = la_next;
    lsum = lsum_next;
}

// One 16x16 tile (t-block TB, s-block SB) of C B^T: rows s = 16SB + 4g + i,
// column t = 16TB + l16 of the MFMA result (fp32).
template <int KN>
__device__ __forceinline__ f32x4 cb_tile(const bf16x8 (&bq)[KN], const bf16x8 (&cq)[KN]) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KN; ++kk) acc = mma(bq[kk], cq[kk], acc);
    return acc;
}

// The explicit form's mask on one C B^T tile, rounded for MFMA.
template <int TB, int SB>
__device__ __forceinline__ bf16x4 mask_tile_hw(const HwDecay& D, const f32x4& acc, int lane) {
    const int l16 = lane & 15, s0 = 16 * SB + 4 * (lane >> 4), t = 16 * TB + l16;
    bf16x4 v;
    if constexpr (TB > SB) {  // off-diagonal: no exponentials
        const f32x4 fa = *(const f32x4*)&D.fa[s0];
        const float f = D.fm[TB * (TB - 1) / 2 + SB] * D.fb[t];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = (bf16)(acc[i] * (fa[i] * f));
    } else {  // diagonal: mask s <= t before the exponential
        const float cst = D.cs2[t];
        const f32x4 css = *(const f32x4*)&D.cs2[s0];
        const f32x4 dts = *(const f32x4*)&D.dt[s0];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool causal = (s0 + i) <= t;
            const float e = fexp2(causal ? cst - css[i] : -INFINITY);
            v[i] = (bf16)(causal ? acc[i] * e * dts[i] : 0.f);
        }
    }
    return v;
}

// Waves per SIMD the registers allow: two (256 VGPRs) for the half-width
// state kernels and for the scans of 8-wave workgroups (which need two per
// SIMD to fit a CU) and of two d_state-64 heads; one (up to 512 VGPRs) for
// full-width waves and the other half-width scans, whose state, fragments and
// outputs of 32 columns need more.
template <int N, int HG, int NPB, int MODE>
constexpr int hw_occupancy() {
    if (NPB == 4) return 1;
    if (MODE == kHwState) return 2;
    return (HG == 4 || (N == 64 && HG == 2)) ? 2 : 1;
}

// Head-wave span kernel; see the file comment.
template <int N, int HG, int NPB, int MODE>
__global__ __launch_bounds__(64 * HG * (4 / NPB), (hw_occupancy<N, HG, NPB, MODE>())) void hw_span_kernel(
    KParams p) {
    using Cf = HwCfg<N, HG, NPB>;
    using Sm = HwSmem<N, HG, NPB, MODE == kHwScan>;
    constexpr int NB = Cf::NB, KN = Cf::KN, WPH = Cf::WPH, NW = Cf::NW;
    constexpr bool SCAN = MODE == kHwScan;
    __shared__ Sm sm;
    touch_args(p);

    // XCD-aware order: consecutive logical blocks (same span, neighbouring
    // head groups, which share B and C) land on the same XCD and its L2.
    // (divisions by the launch's sizes as multiply-highs, set on the host;
    // work items stay below 2^31)
    const Decode& dc = p.dc;
    const int ngrp = dc.ngrp;  // H / HG
    const int64_t bid = blockIdx.x;
    const int64_t logical = (bid % kXcds) * dc.per + bid / kXcds;
    if (logical >= dc.nreal) return;
    const uint32_t lg32 = (uint32_t)logical, rest = fdiv(lg32, dc.by_npg);
    const int pg = (int)(lg32 - rest * (uint32_t)p.npg);
    const uint32_t span32 = fdiv(rest, dc.by_ngrp);
    const int hgi = (int)(rest - span32 * (uint32_t)ngrp);
    const int64_t span = span32;
    const int h0 = hgi * HG;

    int64_t start, len;
    int chunk0, nck;
    if (p.nseq) {
        const int4 e = p.table[span];
        if (e.x < 0) return;
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
    const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
    const int l16 = lane & 15, g = lane >> 4;
    const int q = wave / WPH, wc = wave - q * WPH;
    const int h = h0 + q;
    const int blk0 = wc * NPB;                      // first 16-column block of this wave
    const int nvb = max(0, min(NPB, (pgw - 16 * blk0) / 16));  // blocks inside the headdim

    const int dir = p.reverse ? -1 : 1;
    // token strides (the host keeps them <= 2^24)
    const int XS = (int)p.xs_t, BS = (int)p.bs_t, CS = (int)p.cs_t, DS = (int)p.ds_t;
    const int grp = (int)fdiv((uint32_t)h0, dc.by_hpg);  // h0 G / H
    const bf16* const xg = (const bf16*)p.x + (int64_t)h * p.xs_h + pcol0;
    const bf16* const bg = (const bf16*)p.B + (int64_t)grp * p.bs_g;
    const bf16* const cg = (const bf16*)p.C + (int64_t)grp * p.cs_g;
    const bf16* const dg = (const bf16*)p.d_raw + (int64_t)h * p.ds_h;
    const int64_t cj0 = (int64_t)chunk0 * kChunk;
    const int64_t tb0 = start + (p.reverse ? len - 1 - cj0 : cj0);
    const int dstep = dir * kChunk;
    const int64_t rem0 = len - cj0;
    auto tok0 = [&](int c) -> int64_t { return tb0 + (int64_t)(c * dstep); };
    auto clen_of = [&](int c) -> int { return (int)imin(kChunk, rem0 - (int64_t)c * kChunk); };
    const bf16* const xc0 = xg + tb0 * XS;
    const bf16* const bc0 = bg + tb0 * BS;
    const bf16* const cc0 = cg + tb0 * CS;
    const int64_t xcs = (int64_t)dstep * XS, bcs = (int64_t)dstep * BS, ccs = (int64_t)dstep * CS;

    // Chunk c's tiles: the waves of a head split its X tile, all waves split
    // B and C.  d_raw of a chunk: the head's first wave, one token per lane.
    auto issue_tiles = [&](int c, bf16* __restrict__ xdst, bf16* __restrict__ bdst,
                           bf16* __restrict__ cdst) {
        const int cl = clen_of(c);
        issue_tile<Cf::XIW, 1, Cf::XI>(xdst, xc0 + c * xcs, dir * XS, wc * Cf::XIW, cl, pgw, lane);
        issue_tile<Cf::BIW, NW, Cf::BI>(bdst, bc0 + c * bcs, dir * BS, wave, cl, N, lane);
        if constexpr (SCAN)
            issue_tile<Cf::BIW, NW, Cf::BI>(cdst, cc0 + c * ccs, dir * CS, wave, cl, N, lane);
    };
    auto issue_dr = [&](int c, uint32_t* __restrict__ ddst) {
        const int cl = clen_of(c);
        const void* src = (const void*)(dg + (tok0(c) + dir * (lane < cl ? lane : 0)) * DS);
        __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)ddst, 2, 0, 0);
    };

    // State of this wave's columns, MFMA result order: Hs[nb][b] holds
    // n = 16nb + 4g + i, p = 16(blk0 + b) + l16 (rescaled, see above).
    f32x4 Hs[NB][NPB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int b = 0; b < NPB; ++b) Hs[nb][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16* const sp = (bf16*)p.states + (span * p.H + h) * (int64_t)p.P * N;
    const int pbg = pg * 4 + blk0;  // global 16-column block of this wave's first block
    if constexpr (SCAN) {
        // the state entering the span, as the state pass left it
#pragma unroll
        for (int b = 0; b < NPB; ++b)
            if (b < nvb) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) Hs[nb][b] = load4(sp + state_off(pbg + b, nb, lane, NB));
            }
        // fragment halves that stay zero: tiles above the diagonal (0,1), (2,3)
        for (int i = tid; i < 2 * 64; i += Cf::TH)
            sm.cb[i < 64 ? hw_lslot(0, 0) : hw_lslot(2, 1)][1][i & 63] = bf16x4{};
    }

    // y: this wave's outputs of chunk c at ybase(c) + yoff(tb, b) bytes, with
    // ybase the chunk's lowest token row so every lane offset is >= 0.
    const bf16* const yrow0 = (const bf16*)p.y + (int64_t)h * p.ys_h + pcol0 + 16 * blk0;
    uint32_t yoff[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
        yoff[tb] = (uint32_t)(((p.reverse ? 63 - (16 * tb + l16) : 16 * tb + l16) * p.ys_t + 4 * g) * 2);
    auto ybase = [&](int c) -> const bf16* {
        const int64_t lo = p.reverse ? tok0(c) - (kChunk - 1) : tok0(c);
        const uint64_t a = (uint64_t)(yrow0 + lo * p.ys_t);
        const uint32_t alo = __builtin_amdgcn_readfirstlane((uint32_t)a);
        const uint32_t ahi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
        return (const bf16*)(((uint64_t)ahi << 32) | alo);
    };

    // Prologue: d_raw of chunks 0 and 1, tiles of chunk 0; chunk 0's decay.
    const bool dwave = wc == 0;  // loads its head's d_raw
    float la = 0.f, lsum = 0.f;  // the head's running values before the next chunk formed
    if (dwave) issue_dr(0, sm.dr[0][q]);
    issue_tiles(0, sm.xs[0][q], sm.bs[0], sm.cs[0]);
    if (dwave && nck > 1) issue_dr(1, sm.dr[1][q]);
    vm_wait<0>();
    block_sync();  // d_raw of chunks 0 and 1 is visible to every wave of the head
    hw_decay(sm.dec[0][q], sm.dr[0][q][lane], p.d_init, clen_of(0), lane, la, lsum);

    for (int c = 0; c < nck; ++c) {
        const bool last = c + 1 == nck;
        const int buf = c & 1;
        const int cl = clen_of(c);
        // Chunk c's tiles (and chunk c+1's d_raw, issued before them) are
        // the oldest loads in flight; after them this wave issued only its y
        // stores of chunk c-1: 4 per block, all with some lane active when
        // that chunk was full and every block lies inside the headdim.
        if (SCAN && c > 0 && nvb == NPB) vm_wait<4 * NPB>();
        else vm_wait<0>();
        block_sync();  // chunk c's tiles and decay factors are in LDS, step c-1 is done

        auto body = [&](const bf16* __restrict__ xt, const bf16* __restrict__ bt,
                        const bf16* __restrict__ ct, const uint32_t* __restrict__ drn,
                        bf16* __restrict__ xn, bf16* __restrict__ bn, bf16* __restrict__ cn,
                        uint32_t* __restrict__ drnn, const HwDecay& D, HwDecay& Dn) {
            if (!last) issue_tiles(c + 1, xn, bn, cn);
            if (dwave && c + 2 < nck) issue_dr(c + 2, drnn);
            // the next chunk's decay factors (its d_raw arrived with this
            // chunk's tiles); after the last chunk they are formed from stale
            // d_raw into the free slot and never read
            hw_decay(Dn, drn[lane], p.d_init, clen_of(c + 1), lane, la, lsum);

            const bool slow = __builtin_amdgcn_readfirstlane(__float_as_int(D.slow)) != 0;
            {
                const float hpre = D.hpre;
                if (__builtin_amdgcn_readfirstlane(__float_as_int(hpre)) != __float_as_int(1.f)) {
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                        for (int b = 0; b < NPB; ++b) Hs[nb][b] *= hpre;
                }
            }

            // X^T fragments of this wave's blocks, K = tokens in the order
            // 32kk + 4g + (0..3), 32kk + 16 + 4g + (0..3); scaled to Xs (the
            // update's and the intra-chunk product's operand)
            auto xfrag = [&](int b, int kk) __attribute__((always_inline)) {
                return tok_frag(xt, 32 * kk + 4 * g, 32 * kk + 16 + 4 * g, blk0 + b, lane);
            };
            bf16x8 xw[NPB][2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const f32x4 w0 = *(const f32x4*)&D.w[32 * kk + 4 * g];
                const f32x4 w1 = *(const f32x4*)&D.w[32 * kk + 16 + 4 * g];
#pragma unroll
                for (int b = 0; b < NPB; ++b) {
                    const bf16x8 xf = xfrag(b, kk);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        xw[b][kk][i] = (bf16)((float)xf[i] * w0[i]);
                        xw[b][kk][4 + i] = (bf16)((float)xf[4 + i] * w1[i]);
                    }
                }
            }

            if constexpr (SCAN) {
                // C rows of each t-block (B operand of C B^T and of S^T C^T)
                auto cfrag_tb = [&](int tb, bf16x8(&o)[KN]) __attribute__((always_inline)) {
#pragma unroll
                    for (int kk = 0; kk < KN; ++kk) o[kk] = tile_frag<N>(ct, 16 * tb + l16, kk, g);
                };
                auto bfrag = [&](int sb, bf16x8(&o)[KN]) __attribute__((always_inline)) {
#pragma unroll
                    for (int kk = 0; kk < KN; ++kk) o[kk] = tile_frag<N>(bt, 16 * sb + l16, kk, g);
                };
                // S^T as MFMA A operands (K = d_state in the C fragment order)
                bf16x8 hf[NPB][KN];
#pragma unroll
                for (int b = 0; b < NPB; ++b)
#pragma unroll
                    for (int kk = 0; kk < KN; ++kk) {
                        bf16x4 lo, hi;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            lo[i] = (bf16)Hs[2 * kk][b][i];
                            hi[i] = (bf16)Hs[2 * kk + 1][b][i];
                        }
                        hf[b][kk] = cat<bf16x8, bf16x4>(lo, hi);
                    }
                // per t-block: the inter-chunk term y^T = S^T C^T (state
                // entering chunk c), and this wave's share of the causal C B^T
                // tiles of the block (tile i by wave i % NW)
                f32x4 ye[4][NPB];
                auto tblock = [&](auto tbc) __attribute__((always_inline)) {
                    constexpr int TB = decltype(tbc)::value;
                    bf16x8 cq[KN];
                    cfrag_tb(TB, cq);
#pragma unroll
                    for (int b = 0; b < NPB; ++b) {
                        ye[TB][b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int kk = 0; kk < KN; ++kk) ye[TB][b] = mma(hf[b][kk], cq[kk], ye[TB][b]);
                    }
                    auto share = [&](auto ic_sb) __attribute__((always_inline)) {
                        constexpr int SB = decltype(ic_sb)::value;
                        constexpr int I = TB * (TB + 1) / 2 + SB;  // index in kTileTb / kTileSb
                        if constexpr (SB <= TB) {
                            if (wave == I % NW) {
                                bf16x8 bq[KN];
                                bfrag(SB, bq);
                                const f32x4 acc = cb_tile<KN>(bq, cq);
                                bf16x4 v;
                                const int s0 = 16 * SB + 4 * g, t = 16 * TB + l16;
#pragma unroll
                                for (int i = 0; i < 4; ++i)
                                    v[i] = (bf16)((TB > SB || s0 + i <= t) ? acc[i] : 0.f);
                                sm.cb[hw_lslot(TB, SB >> 1)][SB & 1][lane] = v;
                            }
                        }
                    };
                    share(ic<0>{});
                    share(ic<1>{});
                    share(ic<2>{});
                    share(ic<3>{});
                };
                tblock(ic<0>{});
                tblock(ic<1>{});
                tblock(ic<2>{});
                tblock(ic<3>{});
                block_sync();  // the shared C B^T tiles are complete

                const bf16* const yb = ybase(c);
                if (!slow) {
                    // y^T = fe_t (S^T C^T + Xs^T CB^T), CB^T in K pairs (2kk, 2kk+1)
#pragma unroll
                    for (int tb = 0; tb < 4; ++tb) {
                        const int t = 16 * tb + l16;
                        const bf16x8 l0 = cat<bf16x8, bf16x4>(sm.cb[hw_lslot(tb, 0)][0][lane],
                                                              sm.cb[hw_lslot(tb, 0)][1][lane]);
                        bf16x8 l1 = {};
                        if (tb >= 2)
                            l1 = cat<bf16x8, bf16x4>(sm.cb[hw_lslot(tb, 1)][0][lane],
                                                     sm.cb[hw_lslot(tb, 1)][1][lane]);
                        const float fe = D.fe[t];
#pragma unroll
                        for (int b = 0; b < NPB; ++b) {
                            f32x4 o = mma(xw[b][0], l0, ye[tb][b]);
                            if (tb >= 2) o = mma(xw[b][1], l1, o);
                            store4_masked(yb, yoff[tb] + 32u * b, o * fe, b < nvb && t < cl);
                        }
                    }
                } else {
                    // explicit form: y^T = fe_t S^T C^T + X^T L^T with the
                    // head's decay mask on every C B^T tile (formed here, one
                    // t-block at a time; C, B and X fragments read again from
                    // this chunk's tiles)
                    auto tblock_slow = [&](auto tbc) __attribute__((always_inline)) {
                        constexpr int TB = decltype(tbc)::value;
                        bf16x8 cq[KN];
                        cfrag_tb(TB, cq);
                        bf16x4 v[4];
                        auto tile = [&](auto sbc) __attribute__((always_inline)) {
                            constexpr int SB = decltype(sbc)::value;
                            if constexpr (SB <= TB) {
                                bf16x8 bq[KN];
                                bfrag(SB, bq);
                                v[SB] = mask_tile_hw<TB, SB>(D, cb_tile<KN>(bq, cq), lane);
                            } else {
                                v[SB] = bf16x4{};
                            }
                        };
                        tile(ic<0>{});
                        tile(ic<1>{});
                        tile(ic<2>{});
                        tile(ic<3>{});
                        const int t = 16 * TB + l16;
                        const bf16x8 l0 = cat<bf16x8, bf16x4>(v[0], v[1]);
                        const bf16x8 l1 = cat<bf16x8, bf16x4>(v[2], v[3]);
                        const float fe = D.fe[t];
#pragma unroll
                        for (int b = 0; b < NPB; ++b) {
                            f32x4 o = ye[TB][b] * fe;
                            o = mma(xfrag(b, 0), l0, o);
                            if constexpr (TB >= 2) o = mma(xfrag(b, 1), l1, o);
                            store4_masked(yb, yoff[TB] + 32u * b, o, b < nvb && t < cl);
                        }
                    };
                    tblock_slow(ic<0>{});
                    tblock_slow(ic<1>{});
                    tblock_slow(ic<2>{});
                    tblock_slow(ic<3>{});
                }
            }

            if (!(SCAN && last)) {
                // S' = hpost S + B^T Xs, K = tokens in the X fragment order
                if (slow) {
                    const float hpost = D.hpost;
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                        for (int b = 0; b < NPB; ++b) Hs[nb][b] *= hpost;
                }
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    bf16x8 bq2[2];
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk)
                        bq2[kk] = tok_frag(bt, 32 * kk + 4 * g, 32 * kk + 16 + 4 * g, nb, lane);
#pragma unroll
                    for (int b = 0; b < NPB; ++b)
#pragma unroll
                        for (int kk = 0; kk < 2; ++kk) Hs[nb][b] = mma(bq2[kk], xw[b][kk], Hs[nb][b]);
                }
            }
        };
        body(sm.xs[buf][q], sm.bs[buf], sm.cs[SCAN ? buf : 0], sm.dr[buf ^ 1][q], sm.xs[buf ^ 1][q],
             sm.bs[buf ^ 1], sm.cs[SCAN ? buf ^ 1 : 0], sm.dr[buf][q], sm.dec[buf][q], sm.dec[buf ^ 1][q]);
    }

    if constexpr (!SCAN) {
        // the span's local state H = 2^{la} S, and its decay product
        const HwDecay& D = sm.dec[(nck - 1) & 1][q];
        const float sc = fexp2(D.la);
#pragma unroll
        for (int b = 0; b < NPB; ++b)
            if (b < nvb) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) store4(sp + state_off(pbg + b, nb, lane, NB), Hs[nb][b] * sc);
            }
        if (pg == 0 && wc == 0 && lane == 0) p.decay[span * p.H + h] = fexp2(D.lsum);
    }
}

template <int N, int HG, int NPB, int MODE>
hipError_t launch_hw_t(const KParams& p, hipStream_t s) {
    const int64_t nreal = p.nspan * (p.H / HG) * p.npg;
    if (nreal == 0) return hipSuccess;
    const int64_t grid = (nreal + kXcds - 1) / kXcds * kXcds;
    KParams q = p;
    set_decode(q, HG);
    hipLaunchKernelGGL((hw_span_kernel<N, HG, NPB, MODE>), dim3((unsigned)grid),
                       dim3(HwCfg<N, HG, NPB>::TH), 0, s, q);
    return hipGetLastError();
}

// Full-width waves (npb 4) carry d_state 64; at d_state 128 their state
// and fragments exceed the register file, so only half-width waves are built.
template <int N, int MODE>
hipError_t launch_hw_n(const KParams& p, hipStream_t s) {
    const int hg = MODE == kHwScan ? p.hg_scan : p.hg_state;
    switch (hg * 10 + p.hw_npb) {
        case 12: return launch_hw_t<N, 1, 2, MODE>(p, s);
        case 22: return launch_hw_t<N, 2, 2, MODE>(p, s);
        case 42: return launch_hw_t<N, 4, 2, MODE>(p, s);
    }
    if constexpr (N <= 64) {
        switch (hg * 10 + p.hw_npb) {
            case 14: return launch_hw_t<N, 1, 4, MODE>(p, s);
            case 24: return launch_hw_t<N, 2, 4, MODE>(p, s);
            case 44: return launch_hw_t<N, 4, 4, MODE>(p, s);
        }
    }
    return hipErrorInvalidValue;
}

template <int MODE>
hipError_t launch_hw(const KParams& p, int N, hipStream_t s) {
    switch (N) {
        case 64: return launch_hw_n<64, MODE>(p, s);
        case 128: return launch_hw_n<128, MODE>(p, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

bool hw_supported(int dtype, int N, int hg, int npb) {
    return dtype == 1 && (N == 64 || N == 128) && (hg == 1 || hg == 2 || hg == 4) &&
           (npb == 2 || (npb == 4 && N == 64));
}

size_t hw_lds_bytes(int N, int hg, int npb, bool scan) {
#define SSD_HW_LDS(NN, HH, PP) \
    (scan ? sizeof(HwSmem<NN, HH, PP, true>) : sizeof(HwSmem<NN, HH, PP, false>))
#define SSD_HW_LDS_N(NN)                          \
    switch (hg * 10 + npb) {                      \
        case 14: return SSD_HW_LDS(NN, 1, 4);     \
        case 24: return SSD_HW_LDS(NN, 2, 4);     \
        case 44: return SSD_HW_LDS(NN, 4, 4);     \
        case 12: return SSD_HW_LDS(NN, 1, 2);     \
        case 22: return SSD_HW_LDS(NN, 2, 2);     \
        case 42: return SSD_HW_LDS(NN, 4, 2);     \
    }
    if (!hw_supported(1, N, hg, npb)) return 0;
    if (N == 64) { SSD_HW_LDS_N(64) }
    if (N == 128) { SSD_HW_LDS_N(128) }
#undef SSD_HW_LDS_N
#undef SSD_HW_LDS
    return 0;
}

hipError_t launch_hw_state(const KParams& p, int N, hipStream_t s) { return launch_hw<kHwState>(p, N, s); }
hipError_t launch_hw_scan(const KParams& p, int N, hipStream_t s) { return launch_hw<kHwScan>(p, N, s); }

}  // namespace ssd
