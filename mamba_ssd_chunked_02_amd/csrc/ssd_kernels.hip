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
//   span_state  per (span, head, 64 headdim columns): the span's local state
//               S = sum over its chunks, with the chunk decays, of
//               B^T (w * X) on bf16 MFMA, and the span decay product.
//   state_pass  per (sequence, head, 4 state entries): walks the spans in
//               order, H <- decay * H + S, overwriting each S with the state
//               entering its span; writes final_state.
//   span_scan   per (span, head, 64 columns): starts from the incoming state
//               and, chunk by chunk, forms C B^T, applies the causal decay
//               mask, adds the C Hprev term and writes y, then advances the
//               state (kept in MFMA accumulators) to the next chunk.
// Inside a span the state stays on chip; only span borders go through HBM.
//
// MFMA tiling (v_mfma_f32_16x16x32_bf16; fp32 inputs use 8 x 16x16x4_f32):
// lane l of a wave holds operand row/column l%16 and eight K values chosen by
// l/16; the 16x16 fp32 result holds rows 4*(l/16)+i, column l%16.  A result
// tile pair therefore already is an operand fragment (K = the tile rows), so
// C B^T feeds the intra-chunk product and the state feeds C Hprev with no
// data movement.  Any K order works as long as both operands agree.
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
    static constexpr int EPU = 8;  // elements per 16-byte unit
};
template <> struct Vec<float> {
    using x8 = f32x8;
    using x4 = f32x4;
    static constexpr int EPU = 4;
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

// LDS of one span workgroup.  Tiles indexed [column][token] are the
// token-contracted operands (K = token); [token][n] tiles are n-contracted.
// Every row is padded by 16 bytes so 16-lane column reads spread over banks.
template <typename T, int N, bool SCAN>
struct __attribute__((aligned(16))) Smem {
    static constexpr int PAD = 16 / sizeof(T);
    static constexpr int XP = kChunk + PAD;
    static constexpr int NP = N + PAD;
    static constexpr int YP = kPGroup + PAD;
    static constexpr int SR = SCAN ? kChunk : 1;
    T xT[kPGroup][XP];  // X^T of this workgroup's 64 columns
    T bT[N][XP];        // B^T
    T bn[SR][NP];       // B rows   (scan only)
    T cn[SR][NP];       // C rows   (scan only)
    T yb[SR][YP];       // y tile staged for 16-byte stores (scan only)
    float cs2[kChunk];  // within-chunk cumulative -d, in log2 units
    float dt[kChunk];   // d_s (0 past the end of the sequence)
    float w[kChunk];    // e^{cs_last - cs_s} d_s
};

// Global -> register staging of one chunk (prefetched one chunk ahead).
template <typename T, int N, bool SCAN>
struct Stage {
    static constexpr int EPU = Vec<T>::EPU;
    static constexpr int XPT = (kChunk * kPGroup / EPU + kThreads - 1) / kThreads;
    static constexpr int BUN = kChunk * N / EPU;
    static constexpr int BPT = (BUN + kThreads - 1) / kThreads;
    uint4 xr[XPT];
    uint4 br[BPT];
    uint4 cr[SCAN ? BPT : 1];
    float draw;
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

template <typename T, int N, bool SCAN>
__device__ __forceinline__ void load_chunk(Stage<T, N, SCAN>& st, const KParams& p,
                                           const ChunkPos& cp, int h, int grp,
                                           int pcol0, int upr) {
    using S = Stage<T, N, SCAN>;
    constexpr int EPU = S::EPU;
    const int tid = threadIdx.x;
    const T* xg = (const T*)p.x;
    const T* bg = (const T*)p.B;
    const T* cg = (const T*)p.C;
    const int xun = kChunk * upr;
#pragma unroll
    for (int r = 0; r < S::XPT; ++r) {
        const int u = tid + r * kThreads;
        const int s = u / upr, cu = u - (u / upr) * upr;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (u < xun && s < cp.clen)
            v = *(const uint4*)(xg + (cp.tok(s) * p.H + h) * (int64_t)p.P + pcol0 + cu * EPU);
        st.xr[r] = v;
    }
    constexpr int UPB = N / EPU;  // units per B/C row
#pragma unroll
    for (int r = 0; r < S::BPT; ++r) {
        const int u = tid + r * kThreads;
        const int s = u / UPB, cu = u % UPB;
        uint4 vb = make_uint4(0, 0, 0, 0), vc = make_uint4(0, 0, 0, 0);
        if (u < S::BUN && s < cp.clen) {
            const int64_t off = (cp.tok(s) * p.G + grp) * (int64_t)N + cu * EPU;
            vb = *(const uint4*)(bg + off);
            if (SCAN) vc = *(const uint4*)(cg + off);
        }
        st.br[r] = vb;
        if (SCAN) st.cr[r] = vc;
    }
    if (tid < kChunk) {
        float v = 0.f;
        if (tid < cp.clen) v = (float)((const T*)p.d_raw)[cp.tok(tid) * p.H + h];
        st.draw = v;
    }
}

template <typename T, int N, bool SCAN>
__device__ __forceinline__ void write_chunk(Smem<T, N, SCAN>& sm, const Stage<T, N, SCAN>& st,
                                            const ChunkPos& cp, float d_init, int upr) {
    using S = Stage<T, N, SCAN>;
    constexpr int EPU = S::EPU;
    const int tid = threadIdx.x;
    const int xun = kChunk * upr;
#pragma unroll
    for (int r = 0; r < S::XPT; ++r) {
        const int u = tid + r * kThreads;
        if (u < xun) {
            const int s = u / upr, cu = u - (u / upr) * upr;
            const T* e = (const T*)&st.xr[r];
#pragma unroll
            for (int j = 0; j < EPU; ++j) sm.xT[cu * EPU + j][s] = e[j];
        }
    }
    constexpr int UPB = N / EPU;
#pragma unroll
    for (int r = 0; r < S::BPT; ++r) {
        const int u = tid + r * kThreads;
        if (u < S::BUN) {
            const int s = u / UPB, cu = u % UPB;
            const T* e = (const T*)&st.br[r];
#pragma unroll
            for (int j = 0; j < EPU; ++j) sm.bT[cu * EPU + j][s] = e[j];
            if (SCAN) {
                *(uint4*)&sm.bn[s][cu * EPU] = st.br[r];
                *(uint4*)&sm.cn[s][cu * EPU] = st.cr[r];
            }
        }
    }
    if (tid < kChunk) {
        // step sizes and their within-chunk prefix sum, one lane per token
        const int lane = tid;
        const float dt = lane < cp.clen ? softplus(st.draw + d_init) : 0.f;
        float v = -dt * kLog2e;
#pragma unroll
        for (int off = 1; off < kChunk; off <<= 1) {
            const float o = __shfl_up(v, off, kChunk);
            if (lane >= off) v += o;
        }
        const float last = __shfl(v, kChunk - 1, kChunk);
        sm.cs2[lane] = v;
        sm.dt[lane] = dt;
        sm.w[lane] = exp2f(last - v) * dt;
    }
}

template <typename T, int N, bool SCAN>
__global__ __launch_bounds__(kThreads) void span_kernel(KParams p) {
    using X8 = typename Vec<T>::x8;
    using X4 = typename Vec<T>::x4;
    constexpr int NB = N / 16;           // 16-row blocks of the state
    constexpr int KN = (N + 31) / 32;    // K=32 steps over the state dim
    __shared__ Smem<T, N, SCAN> sm;

    // XCD-aware order: consecutive logical blocks (same span, neighbouring
    // heads, which share B and C) land on the same XCD and its L2.
    const int64_t nreal = p.nspan * p.H * p.npg;
    const int64_t per = (nreal + kXcds - 1) / kXcds;
    const int64_t bid = blockIdx.x;
    const int64_t logical = (bid % kXcds) * per + bid / kXcds;
    if (logical >= nreal) return;
    const int pg = (int)(logical % p.npg);
    const int h = (int)((logical / p.npg) % p.H);
    const int64_t span = logical / ((int64_t)p.npg * p.H);

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

    const int grp = (int)((int64_t)h * p.G / p.H);
    const int pcol0 = pg * kPGroup;
    const int pgw = min(kPGroup, p.P - pcol0);
    const int upr = pgw / Vec<T>::EPU;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l16 = lane & 15, g = lane >> 4;
    const bool active = wave * 16 < pgw;
    const int pw = wave * 16 + l16;  // this lane's column within the group

    f32x4 Hs[NB];
    const int64_t sbase = ((span * p.H + h) * (int64_t)p.P + pcol0 + pw) * N;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        Hs[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (SCAN && active) Hs[nb] = *(const f32x4*)(p.states + sbase + nb * 16 + 4 * g);
    }
    float logdec2 = 0.f;

    ChunkPos cp;
    cp.start = start;
    cp.len = len;
    cp.reverse = p.reverse;
    cp.j0 = (int64_t)chunk0 * kChunk;
    cp.clen = (int)imin(kChunk, len - cp.j0);
    Stage<T, N, SCAN> st;
    load_chunk<T, N, SCAN>(st, p, cp, h, grp, pcol0, upr);

    for (int c = 0; c < nck; ++c) {
        write_chunk<T, N, SCAN>(sm, st, cp, p.d_init, upr);
        __syncthreads();
        ChunkPos nx = cp;
        if (c + 1 < nck) {
            nx.j0 = cp.j0 + kChunk;
            nx.clen = (int)imin(kChunk, len - nx.j0);
            load_chunk<T, N, SCAN>(st, p, nx, h, grp, pcol0, upr);
        }

        if (SCAN && active) {
            // C B^T for the 10 causal 16x16 tiles, stored transposed:
            // cbt[tb][sb] holds rows s = 16sb+4g+i, column t = 16tb+l16.
            f32x4 cbt[10];
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
                for (int sb = 0; sb <= tb; ++sb) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < KN; ++kk) {
                        const int n = 32 * kk + 8 * g;
                        X8 a = {}, b = {};
                        if (N % 32 == 0 || n < N) {
                            a = ld8(&sm.bn[16 * sb + l16][n]);
                            b = ld8(&sm.cn[16 * tb + l16][n]);
                        }
                        acc = mma(a, b, acc);
                    }
                    cbt[tb * (tb + 1) / 2 + sb] = acc;
                }
            }
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                const int t = 16 * tb + l16;
                const float cst = sm.cs2[t];
                f32x4 yi = {0.f, 0.f, 0.f, 0.f}, ye = {0.f, 0.f, 0.f, 0.f};
                // intra-chunk: sum_s L[t][s] X[s][p], L = C B^T * decay * d, s <= t
#pragma unroll
                for (int kk = 0; kk <= tb / 2; ++kk) {
                    X4 half[2];
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const int sb = 2 * kk + hh;
                        X4 v = {};
                        if (sb <= tb) {
                            const int s0 = 16 * sb + 4 * g;
                            const f32x4 css = *(const f32x4*)&sm.cs2[s0];
                            const f32x4 dts = *(const f32x4*)&sm.dt[s0];
                            const f32x4 cb = cbt[tb * (tb + 1) / 2 + sb];
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const bool causal = (s0 + i) <= t;
                                const float e = exp2f(causal ? cst - css[i] : -INFINITY);
                                v[i] = cvt<T>(causal ? cb[i] * e * dts[i] : 0.f);
                            }
                        }
                        half[hh] = v;
                    }
                    const X8 a = cat<X8, X4>(half[0], half[1]);
                    const X8 b = cat<X8, X4>(ld4(&sm.xT[pw][32 * kk + 4 * g]),
                                             ld4(&sm.xT[pw][32 * kk + 16 + 4 * g]));
                    yi = mma(a, b, yi);
                }
                // inter-chunk: sum_n C[t][n] Hprev[n][p]
#pragma unroll
                for (int kk = 0; kk < KN; ++kk) {
                    const int n0 = 32 * kk + 4 * g, n1 = n0 + 16;
                    X4 c0 = {}, c1 = {}, h0 = {}, h1 = {};
                    if (n0 < N) c0 = ld4(&sm.cn[16 * tb + l16][n0]);
                    if (n1 < N) c1 = ld4(&sm.cn[16 * tb + l16][n1]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        h0[i] = cvt<T>(Hs[2 * kk][i]);
                        if (2 * kk + 1 < NB) h1[i] = cvt<T>(Hs[2 * kk + 1][i]);
                    }
                    ye = mma(cat<X8, X4>(c0, c1), cat<X8, X4>(h0, h1), ye);
                }
                const f32x4 csr = *(const f32x4*)&sm.cs2[16 * tb + 4 * g];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sm.yb[16 * tb + 4 * g + i][pw] = cvt<T>(yi[i] + exp2f(csr[i]) * ye[i]);
            }
        }

        if (active) {
            // advance the state over this chunk: H = e^{cs_last} H + B^T (w X)
            const float dec = exp2f(sm.cs2[kChunk - 1]);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) Hs[nb] *= dec;
#pragma unroll
            for (int kk = 0; kk < kChunk / 32; ++kk) {
                const int s0 = 32 * kk + 8 * g;
                const f32x8 ws = ld8(&sm.w[s0]);
                const X8 xv = ld8(&sm.xT[pw][s0]);
                X8 b;
#pragma unroll
                for (int j = 0; j < 8; ++j) b[j] = cvt<T>((float)xv[j] * ws[j]);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) Hs[nb] = mma(ld8(&sm.bT[16 * nb + l16][s0]), b, Hs[nb]);
            }
        }
        if (!SCAN) logdec2 += sm.cs2[kChunk - 1];
        __syncthreads();

        if (SCAN) {
            constexpr int EPU = Vec<T>::EPU;
            T* yg = (T*)p.y;
            for (int u = tid; u < kChunk * upr; u += kThreads) {
                const int t = u / upr, cu = u - (u / upr) * upr;
                if (t < cp.clen)
                    *(uint4*)(yg + cp.tok(t) * p.ys_t + h * p.ys_h + pcol0 + cu * EPU) =
                        *(const uint4*)&sm.yb[t][cu * EPU];
            }
        }
        cp = nx;
    }

    if (!SCAN) {
        if (active) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                *(f32x4*)(p.states + sbase + nb * 16 + 4 * g) = Hs[nb];
        }
        if (pg == 0 && tid == 0) p.decay[span * p.H + h] = exp2f(logdec2);
    }
}

// Walk the spans of one sequence for 4 consecutive state entries [p][n..n+3]:
// replace each span state S_k by the state entering the span and carry
// H <- decay_k H + S_k; H after the last span is the final state.
__global__ __launch_bounds__(256) void state_pass_kernel(KParams p, int N) {
    constexpr int U = 8;
    const int E4 = p.P * N / 4;
    const int64_t S = p.nseq ? p.nseq : p.batch;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (gid >= S * p.H * E4) return;
    const int e4 = (int)(gid % E4);
    const int h = (int)((gid / E4) % p.H);
    const int64_t i = gid / E4 / p.H;
    const int pc = (e4 * 4) / N, n0 = (e4 * 4) % N;
    int64_t s0, s1;
    if (p.nseq) {
        s0 = p.span_off[i];
        s1 = p.span_off[i + 1];
    } else {
        s0 = i * p.sps;
        s1 = s0 + p.sps;
    }
    f32x4 run = {0.f, 0.f, 0.f, 0.f};
    const int64_t sb = ((i * p.H + h) * (int64_t)N + n0) * p.P + pc;  // [S][H][N][P]
    if (p.init) {
#pragma unroll
        for (int j = 0; j < 4; ++j) run[j] = p.init[sb + (int64_t)j * p.P];
    }
    f32x4* st = (f32x4*)p.states;
    for (int64_t k = s0; k < s1; k += U) {
        f32x4 v[U];
        float d[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (k + u < s1) {
                v[u] = st[((k + u) * p.H + h) * E4 + e4];
                d[u] = p.decay[(k + u) * p.H + h];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (k + u < s1) {
                st[((k + u) * p.H + h) * E4 + e4] = run;
                run = d[u] * run + v[u];
            }
        }
    }
    if (p.final_state) {
#pragma unroll
        for (int j = 0; j < 4; ++j) p.final_state[sb + (int64_t)j * p.P] = run[j];
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

template <typename T, int N, bool SCAN>
hipError_t launch_span_t(const KParams& p, hipStream_t s) {
    const int64_t nreal = p.nspan * p.H * p.npg;
    if (nreal == 0) return hipSuccess;
    const int64_t per = (nreal + kXcds - 1) / kXcds;
    hipLaunchKernelGGL((span_kernel<T, N, SCAN>), dim3((unsigned)(per * kXcds)), dim3(kThreads),
                       0, s, p);
    return hipGetLastError();
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

size_t span_lds_bytes(int dtype, int N, bool scan) {
#define SSD_LDS(T, NN) \
    (scan ? sizeof(Smem<T, NN, true>) : sizeof(Smem<T, NN, false>))
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

hipError_t launch_state_pass(const KParams& p, int N, hipStream_t s) {
    const int64_t S = p.nseq ? p.nseq : p.batch;
    const int64_t n = S * p.H * (int64_t)p.P * N / 4;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(state_pass_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, N);
    return hipGetLastError();
}

}  // namespace ssd
