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
#include "ssd_internal.h"

namespace ssd {
namespace {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;

template <typename T> struct Vec;
template <> struct Vec<bf16> {
    using x8 = bf16x8;
    using x4 = bf16x4;
};
template <> struct Vec<float> {
    using x8 = f32x8;
    using x4 = f32x4;
};

__device__ __forceinline__ f32x4 mma(const bf16x8& a, const bf16x8& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(const f32x8& a, const f32x8& b, f32x4 c) {
#pragma unroll
    for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
    return c;
}

// 8 / 4 consecutive elements from 16-byte (x8) / 8-or-16-byte (x4) aligned LDS.
__device__ __forceinline__ bf16x8 ld8(const bf16* p) { return *(const bf16x8*)p; }
__device__ __forceinline__ f32x8 ld8(const float* p) {
    f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
    return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ bf16x4 ld4(const bf16* p) { return *(const bf16x4*)p; }
__device__ __forceinline__ f32x4 ld4(const float* p) { return *(const f32x4*)p; }

template <typename X8, typename X4>
__device__ __forceinline__ X8 cat(const X4& a, const X4& b) {
    X8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) { r[i] = a[i]; r[4 + i] = b[i]; }
    return r;
}

__device__ __forceinline__ float softplus(float z) {
    return fmaxf(z, 0.f) + log1pf(expf(-fabsf(z)));
}

template <typename T>
__device__ __forceinline__ T cvt(float v) { return (T)v; }

__device__ __forceinline__ int64_t imin(int64_t a, int64_t b) { return a < b ? a : b; }

// Four consecutive outputs of one token: 8-byte (bf16) or 16-byte (fp32) store.
__device__ __forceinline__ void store4(bf16* p, const f32x4& v) {
    bf16x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = (bf16)v[i];
    *(bf16x4*)p = o;
}
__device__ __forceinline__ void store4(float* p, const f32x4& v) { *(f32x4*)p = v; }

// Four consecutive span-state values (states are stored in the input type).
__device__ __forceinline__ f32x4 load4(const bf16* p) {
    const bf16x4 v = *(const bf16x4*)p;
    return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
__device__ __forceinline__ f32x4 load4(const float* p) { return *(const f32x4*)p; }

// Compile-time shape of one span workgroup: HG heads (sharing one B/C group)
// x 64 headdim columns, one 16-column block per wave.
template <typename T, int N, int HG>
struct Cfg {
    static constexpr int NB = N / 16;            // 16-row blocks of the state
    static constexpr int KN = (N + 31) / 32;     // K=32 steps over the state dim
    static constexpr int EPU = 16 / sizeof(T);   // elements per 16-byte unit
    static constexpr int XP = kPGroup + EPU;     // row pitch of X tiles (elements)
    static constexpr int NP = N + EPU;           // row pitch of B / C tiles
    static constexpr int XU = kPGroup / EPU;     // 16-byte units per X row
    static constexpr int BU = N / EPU;           // 16-byte units per B / C row
    static constexpr int XIT = kChunk * XU / kThreads;
    static constexpr int BIT = (kChunk * BU + kThreads - 1) / kThreads;
};

// Heads per workgroup: the span_state kernel keeps HG states of N x 16 per
// wave in registers, span_scan also the output tiles, so it carries fewer.
constexpr int heads_state(int N) { return N <= 128 ? 4 : 2; }
constexpr int heads_scan(int N) { return N <= 128 ? 2 : 1; }

// Wave index within the workgroup as a scalar, so branches on it stay uniform.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Raw v_exp_f32: every argument here is <= 0, results below 2^-126 flush to 0.
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Token-contracted MFMA fragment from a natural [token][col] LDS tile: this
// lane's column c0 + lane%16 at tokens r0..r0+3 (slots 0-3) and r1..r1+3
// (slots 4-7); r0, r1 are the same for the 16 lanes of a group.  bf16 uses
// the gfx950 transposing read (ds_read_b64_tr_b16): lane i of a 16-lane
// group receives, in slot k, element i%4 of the 8 bytes addressed by lane
// 4k + i/4 of the group, so lane j addresses row r + j/4, columns
// c0 + 4(j%4)..+3.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x4 ldtr(const bf16* p) {
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(p));
    return __builtin_bit_cast(bf16x4, v);
}
__device__ __forceinline__ bf16x8 tok_frag(const bf16* tile, int pitch, int r0, int r1, int c0,
                                           int lane) {
    const int j = lane & 15;
    const bf16* q = tile + (j >> 2) * pitch + c0 + 4 * (j & 3);
    return cat<bf16x8, bf16x4>(ldtr(q + r0 * pitch), ldtr(q + r1 * pitch));
}
__device__ __forceinline__ f32x8 tok_frag(const float* tile, int pitch, int r0, int r1, int c0,
                                          int lane) {
    const float* q = tile + c0 + (lane & 15);
    f32x8 r;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        r[k] = q[(r0 + k) * pitch];
        r[4 + k] = q[(r1 + k) * pitch];
    }
    return r;
}

// Per-head, per-chunk decay factors (cs = within-chunk cumulative -d in log2
// units, c_k = cs at the last token of 16-token block k-1, c_0 = 0).  For s in
// block sb < tb and t in block tb,
//   e^{cs_t - cs_s} d_s = fa_s * fm(tb, sb) * fb_t,
//   fa_s = 2^{c_{sb+1} - cs_s} d_s,  fm = 2^{c_tb - c_{sb+1}},  fb_t = 2^{cs_t - c_tb},
// each factor <= 1, so off-diagonal mask tiles need no exponentials.
struct Decay {
    float cs2[kChunk];  // cs
    float dt[kChunk];   // d_s (0 past the end of the sequence)
    float w[kChunk];    // 2^{cs_last - cs_s} d_s   (state update weights)
    float fa[kChunk];
    float fb[kChunk];
    float fe[kChunk];   // 2^{cs_t}
    float fm[8];        // block pairs (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
};

// Fragment slots of the masked C B^T, the B operand of y^T += X^T L^T:
// (tb, kk) -> tb=0: 0, tb=1: 1, tb=2: 2+kk, tb=3: 4+kk.
__device__ __forceinline__ constexpr int lslot(int tb, int kk) {
    return tb == 0 ? 0 : (tb == 1 ? 1 : (tb == 2 ? 2 + kk : 4 + kk));
}

// Span states are kept in MFMA result order so each wave moves 64 contiguous
// 4-value groups: within one (span, head) block of P*N values, state entry
// (n, p) with p = 16*pb + l, n = 16*nb + 4*g + i sits at
// ((pb*NB + nb)*64 + 16*g + l)*4 + i.
__device__ __forceinline__ int64_t state_off(int pb, int nb, int lane, int NB) {
    return ((int64_t)(pb * NB + nb) * 64 + lane) * 4;
}

// LDS of one span workgroup: natural [token][column] tiles, rows padded by
// 16 bytes.
template <typename T, int N, int HG, bool SCAN>
struct __attribute__((aligned(16))) Smem {
    using C = Cfg<T, N, HG>;
    using X8 = typename Vec<T>::x8;
    T xs[HG][kChunk][C::XP];          // X of every head, this group's 64 columns
    T bs[kChunk][C::NP];              // B
    T cs[SCAN ? kChunk : 1][C::NP];   // C                               (scan only)
    X8 lf[SCAN ? HG : 1][6][64];      // masked C B^T fragments per head (scan only)
    Decay dec[HG];
};

// Global -> register staging of one chunk, prefetched one chunk ahead; 16-byte
// units, consecutive lanes along a row.
template <typename T, int N, int HG, bool SCAN>
struct Stage {
    using C = Cfg<T, N, HG>;
    uint4 xr[HG][C::XIT];
    uint4 br[C::BIT];
    uint4 cr[SCAN ? C::BIT : 1];
    float draw;  // d_raw of token lane for head `wave`
};

struct ChunkPos {
    int64_t start, len, j0;  // sequence start/length, first logical token
    int clen;                // tokens of this chunk (<= 64)
    int reverse;
    __device__ __forceinline__ int64_t tok(int s) const {
        const int64_t j = j0 + s;
        return start + (reverse ? (len - 1 - j) : j);
    }
};

// Issue every global load of one chunk into registers.
template <typename T, int N, int HG, bool SCAN>
__device__ __forceinline__ void load_chunk(Stage<T, N, HG, SCAN>& st, const KParams& p,
                                           const ChunkPos& cp, int h0, int nh, int grp,
                                           int pcol0, int xun) {
    using C = Cfg<T, N, HG>;
    const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
    const int64_t HP = (int64_t)p.H * p.P;
    const T* xg = (const T*)p.x + (int64_t)h0 * p.P + pcol0;
#pragma unroll
    for (int it = 0; it < C::XIT; ++it) {
        const int u = tid + it * kThreads;
        const int s = u / C::XU, c = u % C::XU;
        const bool ok = c < xun && s < cp.clen;
        const T* row = xg + (ok ? cp.tok(s) : 0) * HP + c * C::EPU;
#pragma unroll
        for (int hh = 0; hh < HG; ++hh) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (ok && hh < nh) v = *(const uint4*)(row + hh * p.P);
            st.xr[hh][it] = v;
        }
    }
    const T* bg = (const T*)p.B + (int64_t)grp * N;
    const T* cg = (const T*)p.C + (int64_t)grp * N;
    const int64_t GN = (int64_t)p.G * N;
#pragma unroll
    for (int it = 0; it < C::BIT; ++it) {
        const int u = tid + it * kThreads;
        const int s = u / C::BU, c = u % C::BU;
        uint4 vb = make_uint4(0, 0, 0, 0), vc = make_uint4(0, 0, 0, 0);
        if (u < kChunk * C::BU && s < cp.clen) {
            const int64_t off = cp.tok(s) * GN + c * C::EPU;
            vb = *(const uint4*)(bg + off);
            if (SCAN) vc = *(const uint4*)(cg + off);
        }
        st.br[it] = vb;
        if (SCAN) st.cr[it] = vc;
    }
    {
        const int hh = wave;  // wave hh holds head hh's d_raw, one token per lane
        float v = 0.f;
        if (hh < nh && lane < cp.clen) v = (float)((const T*)p.d_raw)[cp.tok(lane) * p.H + h0 + hh];
        st.draw = v;
    }
}

// Registers -> LDS for one chunk; wave hh also forms head hh's decay factors.
template <typename T, int N, int HG, bool SCAN>
__device__ __forceinline__ void write_chunk(Smem<T, N, HG, SCAN>& sm,
                                            const Stage<T, N, HG, SCAN>& st,
                                            const ChunkPos& cp, float d_init, int nh) {
    using C = Cfg<T, N, HG>;
    const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
#pragma unroll
    for (int it = 0; it < C::XIT; ++it) {
        const int u = tid + it * kThreads;
        const int s = u / C::XU, c = u % C::XU;
#pragma unroll
        for (int hh = 0; hh < HG; ++hh)
            if (hh < nh) *(uint4*)&sm.xs[hh][s][c * C::EPU] = st.xr[hh][it];
    }
#pragma unroll
    for (int it = 0; it < C::BIT; ++it) {
        const int u = tid + it * kThreads;
        const int s = u / C::BU, c = u % C::BU;
        if (u < kChunk * C::BU) {
            *(uint4*)&sm.bs[s][c * C::EPU] = st.br[it];
            if (SCAN) *(uint4*)&sm.cs[s][c * C::EPU] = st.cr[it];
        }
    }
    if (wave < nh && wave < HG) {
        // step sizes, their within-chunk prefix sum and the decay factors of
        // head `wave`, one lane per token
        Decay& D = sm.dec[wave];
        const float dt = lane < cp.clen ? softplus(st.draw + d_init) : 0.f;
        float v = -dt * kLog2e;
#pragma unroll
        for (int off = 1; off < kChunk; off <<= 1) {
            const float o = __shfl_up(v, off, kChunk);
            if (lane >= off) v += o;
        }
        const float c1 = __shfl(v, 15, kChunk), c2 = __shfl(v, 31, kChunk);
        const float c3 = __shfl(v, 47, kChunk), c4 = __shfl(v, 63, kChunk);
        const int sb = lane >> 4;
        const float cbeg = sb == 0 ? 0.f : (sb == 1 ? c1 : (sb == 2 ? c2 : c3));
        const float cend = sb == 0 ? c1 : (sb == 1 ? c2 : (sb == 2 ? c3 : c4));
        D.cs2[lane] = v;
        D.dt[lane] = dt;
        D.w[lane] = fexp2(c4 - v) * dt;
        D.fa[lane] = fexp2(cend - v) * dt;
        D.fb[lane] = fexp2(v - cbeg);
        D.fe[lane] = fexp2(v);
        if (lane < 6) {
            // (tb, sb) = (1,0) (2,0) (2,1) (3,0) (3,1) (3,2): 2^{c_tb - c_{sb+1}}
            const float ct = lane == 0 ? c1 : (lane < 3 ? c2 : c3);
            const float cs = (lane == 0 || lane == 1 || lane == 3) ? c1 : ((lane == 2 || lane == 4) ? c2 : c3);
            D.fm[lane] = fexp2(ct - cs);
        }
    }
}

// C B^T tiles of s-block SB (t-blocks tb >= SB: row s = 16*SB + 4g + i,
// column t = 16*tb + l16 of the MFMA result), then for every head the tiles
// times the decay mask, rounded, as halves of the intra-chunk B fragments.
template <int SB, typename T, int N, int HG, bool SCAN>
__device__ __forceinline__ void mask_phase(Smem<T, N, HG, SCAN>& sm, int nh, int lane) {
    using X8 = typename Vec<T>::x8;
    using X4 = typename Vec<T>::x4;
    constexpr int KN = Cfg<T, N, HG>::KN;
    const int l16 = lane & 15, g = lane >> 4;
    X8 a[KN];  // B rows 16*SB + l16, n = 32kk + 8g ..
#pragma unroll
    for (int kk = 0; kk < KN; ++kk) {
        const int n = 32 * kk + 8 * g;
        a[kk] = X8{};
        if (N % 32 == 0 || n < N) a[kk] = ld8(&sm.bs[16 * SB + l16][n]);
    }
    f32x4 cbt[4];
#pragma unroll
    for (int tb = SB; tb < 4; ++tb) {
        X8 b[KN];
#pragma unroll
        for (int kk = 0; kk < KN; ++kk) {
            const int n = 32 * kk + 8 * g;
            b[kk] = X8{};
            if (N % 32 == 0 || n < N) b[kk] = ld8(&sm.cs[16 * tb + l16][n]);
        }
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KN; ++kk) acc = mma(a[kk], b[kk], acc);
        cbt[tb] = acc;
    }
    const int s0 = 16 * SB + 4 * g;
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
        if (hh < nh) {
            const Decay& D = sm.dec[hh];
            const f32x4 fa = *(const f32x4*)&D.fa[s0];
#pragma unroll
            for (int tb = SB + 1; tb < 4; ++tb) {  // off-diagonal: no exponentials
                const float f = D.fm[tb * (tb - 1) / 2 + SB] * D.fb[16 * tb + l16];
                X4 v;
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = cvt<T>(cbt[tb][i] * (fa[i] * f));
                *((X4*)&sm.lf[hh][lslot(tb, SB >> 1)][lane] + (SB & 1)) = v;
            }
            {  // diagonal tile: mask s <= t before the exponential
                const int t = 16 * SB + l16;
                const float cst = D.cs2[t];
                const f32x4 css = *(const f32x4*)&D.cs2[s0];
                const f32x4 dts = *(const f32x4*)&D.dt[s0];
                X4 v;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool causal = (s0 + i) <= t;
                    const float e = fexp2(causal ? cst - css[i] : -INFINITY);
                    v[i] = cvt<T>(causal ? cbt[SB][i] * e * dts[i] : 0.f);
                }
                *((X4*)&sm.lf[hh][lslot(SB, SB >> 1)][lane] + (SB & 1)) = v;
            }
        }
    }
}

// Two workgroups per CU when their LDS fits in the 160 KB of a gfx950 CU.
template <typename T, int N, int HG, bool SCAN>
constexpr int span_occupancy() { return 2 * sizeof(Smem<T, N, HG, SCAN>) <= 160 * 1024 ? 2 : 1; }

template <typename T, int N, int HG, bool SCAN>
__global__ __launch_bounds__(kThreads, (span_occupancy<T, N, HG, SCAN>())) void span_kernel(
    KParams p) {
    using Cf = Cfg<T, N, HG>;
    using X8 = typename Vec<T>::x8;
    using X4 = typename Vec<T>::x4;
    constexpr int NB = Cf::NB, KN = Cf::KN;
    __shared__ Smem<T, N, HG, SCAN> sm;

    // XCD-aware order: consecutive logical blocks (same span, neighbouring
    // head groups, which share B and C) land on the same XCD and its L2.
    const int hg = SCAN ? p.hg_scan : p.hg_state;
    const int ngrp = (p.H + hg - 1) / hg;
    const int64_t nreal = p.nspan * ngrp * p.npg;
    const int64_t per = (nreal + kXcds - 1) / kXcds;
    const int64_t bid = blockIdx.x;
    const int64_t logical = (bid % kXcds) * per + bid / kXcds;
    if (logical >= nreal) return;
    const int pg = (int)(logical % p.npg);
    const int hgi = (int)((logical / p.npg) % ngrp);
    const int64_t span = logical / ((int64_t)p.npg * ngrp);
    const int h0 = hgi * hg;
    const int nh = min(hg, p.H - h0);  // hg <= HG divides H/G: one B/C group

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
        const int64_t seq = span / p.sps;
        const int kin = (int)(span - seq * p.sps);
        start = seq * p.L;
        len = p.L;
        const int64_t nch = (len + kChunk - 1) / kChunk;
        chunk0 = kin * p.K;
        nck = (int)imin(p.K, nch - chunk0);
    }
    if (nck <= 0) return;

    const int pcol0 = pg * kPGroup;
    const int pgw = min(kPGroup, p.P - pcol0);
    const int xun = pgw / Cf::EPU;
    const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
    const int l16 = lane & 15, g = lane >> 4;
    const bool active = wave * 16 < pgw;
    const int pb = pg * kWaves + wave;  // this wave's 16-column block of headdim

    f32x4 Hs[HG][NB];
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
        const T* sb = (const T*)p.states + (span * p.H + h0 + hh) * (int64_t)p.P * N;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            Hs[hh][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (SCAN && active && hh < nh) Hs[hh][nb] = load4(sb + state_off(pb, nb, lane, NB));
        }
    }
    float logdec2 = 0.f;  // wave hh: sum of head hh's chunk log2-decays

    if (SCAN) {
        // mask fragment halves that stay zero: tiles above the diagonal
        // (tb, sb) = (0, 1) and (2, 3)
        for (int i = tid; i < HG * 2 * 64; i += kThreads) {
            const int hh = i / 128, k = (i / 64) & 1, l = i & 63;
            X4* dst = (X4*)&sm.lf[hh][k ? lslot(2, 1) : lslot(0, 0)][l] + 1;
            *dst = X4{};
        }
    }

    ChunkPos cp;
    cp.start = start;
    cp.len = len;
    cp.reverse = p.reverse;
    cp.j0 = (int64_t)chunk0 * kChunk;
    cp.clen = (int)imin(kChunk, len - cp.j0);
    const int grp = (int)((int64_t)h0 * p.G / p.H);
    Stage<T, N, HG, SCAN> st;
    load_chunk<T, N, HG, SCAN>(st, p, cp, h0, nh, grp, pcol0, xun);
    T* const yg = (T*)p.y + pcol0 + wave * 16 + 4 * g;
    const int wc = wave * 16;  // this wave's first column in the X tiles

    for (int c = 0; c < nck; ++c) {
        const bool last_chunk = c + 1 == nck;
        const bool need_update = !SCAN || !last_chunk;
        __syncthreads();  // previous chunk's tiles are no longer read
        write_chunk<T, N, HG, SCAN>(sm, st, cp, p.d_init, nh);
        __syncthreads();
        ChunkPos nx = cp;
        int64_t yo[4];
        if (SCAN) {
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                const int t = 16 * tb + l16;
                yo[tb] = t < cp.clen ? cp.tok(t) * p.ys_t : -1;
            }
        }
        if (!last_chunk) {
            nx.j0 = cp.j0 + kChunk;
            nx.clen = (int)imin(kChunk, len - nx.j0);
            load_chunk<T, N, HG, SCAN>(st, p, nx, h0, nh, grp, pcol0, xun);
        }

        if constexpr (SCAN) {
            // C B^T tiles of s-block `wave`, then every head's masked fragments
            switch (wave) {
                case 0: mask_phase<0, T, N, HG, SCAN>(sm, nh, lane); break;
                case 1: mask_phase<1, T, N, HG, SCAN>(sm, nh, lane); break;
                case 2: mask_phase<2, T, N, HG, SCAN>(sm, nh, lane); break;
                default: mask_phase<3, T, N, HG, SCAN>(sm, nh, lane); break;
            }
            __syncthreads();
        }

        if (active) {
#pragma unroll
            for (int hh = 0; hh < HG; ++hh) {
                if (hh < nh) {
                    const Decay& D = sm.dec[hh];
                    const T* xt = &sm.xs[hh][0][0];
                    if (SCAN) {
                        const int h = h0 + hh;
                        X8 hf[KN];  // this head's state as the A operand of H^T C^T
#pragma unroll
                        for (int kk = 0; kk < KN; ++kk) {
                            X4 lo, hi = {};
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                lo[i] = cvt<T>(Hs[hh][2 * kk][i]);
                                if (2 * kk + 1 < NB) hi[i] = cvt<T>(Hs[hh][2 * kk + 1][i]);
                            }
                            hf[kk] = cat<X8, X4>(lo, hi);
                        }
                        // X^T fragments in the K order of the mask tiles:
                        // tokens 32kk + 4g + (0..3) and 32kk + 16 + 4g + (0..3)
                        X8 xf[2], lfr[6];
#pragma unroll
                        for (int kk = 0; kk < 2; ++kk)
                            xf[kk] = tok_frag(xt, Cf::XP, 32 * kk + 4 * g, 32 * kk + 16 + 4 * g, wc,
                                              lane);
#pragma unroll
                        for (int j = 0; j < 6; ++j) lfr[j] = sm.lf[hh][j][lane];
                        // intra-chunk: y^T += X^T L^T (causal fragments only)
                        f32x4 yi[4], ye[4];
                        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                        yi[0] = mma(xf[0], lfr[lslot(0, 0)], z);
                        yi[1] = mma(xf[0], lfr[lslot(1, 0)], z);
                        yi[2] = mma(xf[0], lfr[lslot(2, 0)], z);
                        yi[3] = mma(xf[0], lfr[lslot(3, 0)], z);
                        yi[2] = mma(xf[1], lfr[lslot(2, 1)], yi[2]);
                        yi[3] = mma(xf[1], lfr[lslot(3, 1)], yi[3]);
                        // inter-chunk: y^T += H^T C^T, four independent chains
#pragma unroll
                        for (int tb = 0; tb < 4; ++tb) ye[tb] = z;
#pragma unroll
                        for (int kk = 0; kk < KN; ++kk) {
                            const int n0 = 32 * kk + 4 * g, n1 = n0 + 16;
                            X8 cf[4];
#pragma unroll
                            for (int tb = 0; tb < 4; ++tb) {
                                X4 c0 = {}, c1 = {};
                                if (N % 32 == 0 || n0 < N) c0 = ld4(&sm.cs[16 * tb + l16][n0]);
                                if (N % 32 == 0 || n1 < N) c1 = ld4(&sm.cs[16 * tb + l16][n1]);
                                cf[tb] = cat<X8, X4>(c0, c1);
                            }
#pragma unroll
                            for (int tb = 0; tb < 4; ++tb) ye[tb] = mma(hf[kk], cf[tb], ye[tb]);
                        }
                        T* const yh = yg + (int64_t)h * p.ys_h;
#pragma unroll
                        for (int tb = 0; tb < 4; ++tb) {
                            const float sc = D.fe[16 * tb + l16];
                            f32x4 o;
#pragma unroll
                            for (int i = 0; i < 4; ++i) o[i] = yi[tb][i] + sc * ye[tb][i];
                            if (yo[tb] >= 0) store4(yh + yo[tb], o);
                        }
                    }
                    if (need_update) {
                        // advance the state over this chunk: H = e^{cs_last} H + B^T (w X)
                        const float decay = D.fe[kChunk - 1];
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb) Hs[hh][nb] *= decay;
#pragma unroll
                        for (int kk = 0; kk < kChunk / 32; ++kk) {
                            const int s0 = 32 * kk + 8 * g;  // tokens s0 .. s0+7
                            const f32x8 ws = ld8(&D.w[s0]);
                            const X8 xv = tok_frag(xt, Cf::XP, s0, s0 + 4, wc, lane);
                            X8 b, bt[NB];
#pragma unroll
                            for (int nb = 0; nb < NB; ++nb)
                                bt[nb] = tok_frag(&sm.bs[0][0], Cf::NP, s0, s0 + 4, 16 * nb, lane);
#pragma unroll
                            for (int j = 0; j < 8; ++j) b[j] = cvt<T>((float)xv[j] * ws[j]);
#pragma unroll
                            for (int nb = 0; nb < NB; ++nb) Hs[hh][nb] = mma(bt[nb], b, Hs[hh][nb]);
                        }
                    }
                }
            }
        }
        if (!SCAN && wave < nh) logdec2 += sm.dec[wave].cs2[kChunk - 1];
        cp = nx;
    }

    if (!SCAN) {
#pragma unroll
        for (int hh = 0; hh < HG; ++hh) {
            if (hh < nh && active) {
                T* sb = (T*)p.states + (span * p.H + h0 + hh) * (int64_t)p.P * N;
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) store4(sb + state_off(pb, nb, lane, NB), Hs[hh][nb]);
            }
        }
        if (pg == 0 && wave < nh && lane == 0) p.decay[span * p.H + h0 + wave] = fexp2(logdec2);
    }
}

// Walk the spans of one sequence for V = 16 bytes of consecutive stored
// state entries: replace each span state S_k (input type) by the state
// entering the span and carry H <- decay_k H + S_k in fp32; H after the last
// span is the final state.  Stored entry o of a (span, head) block holds
// state (n, p) as laid out by state_off(); init/final are [N][P].
template <typename TS>
__global__ __launch_bounds__(256) void state_pass_kernel(KParams p) {
    constexpr int U = 8;                 // spans in flight per thread
    constexpr int V = 16 / sizeof(TS);   // state entries per thread
    typedef TS TSV __attribute__((ext_vector_type(V)));
    typedef float FV __attribute__((ext_vector_type(V)));
    const int N = p.N, NB = p.N / 16;
    const int EV = p.P * N / V;
    const int64_t S = p.nseq ? p.nseq : p.batch;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (gid >= S * p.H * EV) return;
    const int ev = (int)(gid % EV);
    const int h = (int)((gid / EV) % p.H);
    const int64_t i = gid / EV / p.H;
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
        const int n = 16 * (q % NB) + 4 * (lane >> 4) + (o & 3);
        const int pp = 16 * (q / NB) + (lane & 15);
        idx[j] = n * p.P + pp;
    }
    const int64_t hb = (i * p.H + h) * (int64_t)N * p.P;
    FV run = {};
    if (p.init) {
#pragma unroll
        for (int j = 0; j < V; ++j) run[j] = p.init[hb + idx[j]];
    }
    TSV* st = (TSV*)p.states;
    for (int64_t k = s0; k < s1; k += U) {
        TSV v[U];
        float d[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (k + u < s1) {
                v[u] = st[((k + u) * p.H + h) * EV + ev];
                d[u] = p.decay[(k + u) * p.H + h];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (k + u < s1) {
                TSV o;
#pragma unroll
                for (int j = 0; j < V; ++j) o[j] = (TS)run[j];
                st[((k + u) * p.H + h) * EV + ev] = o;
#pragma unroll
                for (int j = 0; j < V; ++j) run[j] = d[u] * run[j] + (float)v[u][j];
            }
        }
    }
    if (p.final_state) {
#pragma unroll
        for (int j = 0; j < V; ++j) p.final_state[hb + idx[j]] = run[j];
    }
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

template <typename T, int N, int HG, bool SCAN>
hipError_t launch_span_hg(const KParams& p, int hg, hipStream_t s) {
    const int64_t nreal = p.nspan * ((p.H + hg - 1) / hg) * p.npg;
    if (nreal == 0) return hipSuccess;
    const int64_t per = (nreal + kXcds - 1) / kXcds;
    hipLaunchKernelGGL((span_kernel<T, N, HG, SCAN>), dim3((unsigned)(per * kXcds)),
                       dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

// Instantiated for 1, 2 and 4 heads per workgroup, up to the most the kernel
// can carry at this d_state.
template <typename T, int N, bool SCAN>
hipError_t launch_span_t(const KParams& p, hipStream_t s) {
    constexpr int MAXH = SCAN ? heads_scan(N) : heads_state(N);
    const int hg = SCAN ? p.hg_scan : p.hg_state;
    if (hg == 1) return launch_span_hg<T, N, 1, SCAN>(p, 1, s);
    if (hg == 2 && MAXH >= 2) return launch_span_hg<T, N, (MAXH >= 2 ? 2 : 1), SCAN>(p, 2, s);
    if (hg == 4 && MAXH >= 4) return launch_span_hg<T, N, (MAXH >= 4 ? 4 : 1), SCAN>(p, 4, s);
    return hipErrorInvalidValue;
}

template <bool SCAN>
hipError_t launch_span(const KParams& p, int dtype, int N, hipStream_t s) {
    if (dtype == 1) {
        switch (N) {
            case 16: return launch_span_t<bf16, 16, SCAN>(p, s);
            case 32: return launch_span_t<bf16, 32, SCAN>(p, s);
            case 64: return launch_span_t<bf16, 64, SCAN>(p, s);
            case 128: return launch_span_t<bf16, 128, SCAN>(p, s);
            case 256: return launch_span_t<bf16, 256, SCAN>(p, s);
        }
    } else {
        switch (N) {
            case 16: return launch_span_t<float, 16, SCAN>(p, s);
            case 32: return launch_span_t<float, 32, SCAN>(p, s);
            case 64: return launch_span_t<float, 64, SCAN>(p, s);
            case 128: return launch_span_t<float, 128, SCAN>(p, s);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace

int span_max_heads(int N, bool scan) { return scan ? heads_scan(N) : heads_state(N); }

size_t span_lds_bytes(int dtype, int N, bool scan) {
#define SSD_LDS(T, NN)                                                 \
    (scan ? sizeof(Smem<T, NN, heads_scan(NN), true>)                  \
          : sizeof(Smem<T, NN, heads_state(NN), false>))
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

hipError_t launch_span_state(const KParams& p, int dtype, int N, hipStream_t s) {
    return launch_span<false>(p, dtype, N, s);
}

hipError_t launch_span_scan(const KParams& p, int dtype, int N, hipStream_t s) {
    return launch_span<true>(p, dtype, N, s);
}

hipError_t launch_state_pass(const KParams& p, int dtype, hipStream_t s) {
    const int64_t S = p.nseq ? p.nseq : p.batch;
    const int V = dtype == 1 ? 8 : 4;
    const int64_t n = S * p.H * (int64_t)p.P * p.N / V;
    if (n == 0) return hipSuccess;
    const dim3 grid((unsigned)((n + 255) / 256));
    if (dtype == 1)
        hipLaunchKernelGGL(state_pass_kernel<bf16>, grid, dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL(state_pass_kernel<float>, grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace ssd
