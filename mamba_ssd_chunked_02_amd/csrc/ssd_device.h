// Device helpers shared by the span kernels (ssd_kernels.hip) and the
// head-wave kernels (ssd_hw_kernels.hip): vector types, MFMA wrappers, the
// column-blocked LDS tile layout with its direct global->LDS loads and
// fragment reads, explicit waits, the wavefront prefix sum and the
// per-chunk decay factors.  Internal; each translation unit gets its own
// copy (anonymous namespace).
#pragma once

#include "ssd_internal.h"

namespace ssd {
namespace {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
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

template <typename T>
__device__ __forceinline__ T cvt(float v) { return (T)v; }

__device__ __forceinline__ int64_t imin(int64_t a, int64_t b) { return a < b ? a : b; }
constexpr int imin_c(int a, int b) { return a < b ? a : b; }

// Four consecutive outputs of one token: 8-byte (bf16) or 16-byte (fp32) store.
__device__ __forceinline__ void store4(bf16* p, const f32x4& v) {
    bf16x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = (bf16)v[i];
    *(bf16x4*)p = o;
}
__device__ __forceinline__ void store4(float* p, const f32x4& v) { *(f32x4*)p = v; }

// The same stores issued as inline assembly.  The compiler's wait insertion
// treats pending stores and loads on the vector-memory counter as unordered
// and would then wait for every outstanding load (the prefetched tiles
// included) before the next use of a loaded register; stores it does not see
// leave its waits for loads exact.  Loads still retire in issue order, so
// every wait it computes stays sufficient.  The s_nop covers the one wait
// state a store of more than 8 bytes needs before its data registers are
// overwritten.
__device__ __forceinline__ void store4_async(bf16* p, const f32x4& v) {
    bf16x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = (bf16)v[i];
    asm volatile("global_store_dwordx2 %0, %1, off" ::"v"(p), "v"(o) : "memory");
}
__device__ __forceinline__ void store4_async(float* p, const f32x4& v) {
    asm volatile("global_store_dwordx4 %0, %1, off\n\ts_nop 0" ::"v"(p), "v"(v) : "memory");
}

// Four consecutive span-state values (states are stored in the input type).
__device__ __forceinline__ f32x4 load4(const bf16* p) {
    const bf16x4 v = *(const bf16x4*)p;
    return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
__device__ __forceinline__ f32x4 load4(const float* p) { return *(const f32x4*)p; }


// Wave index within the workgroup as a scalar, so branches on it stay uniform.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Inclusive prefix sum over the 64 lanes of a wave with DPP row shifts and
// row broadcasts (no LDS round trips).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float v) {
    const int t = __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, false);
    return v + __int_as_float(t);
}
__device__ __forceinline__ float wave_prefix_sum(float v) {
    v = dpp_add<0x111, 0xf>(v);  // row_shr:1
    v = dpp_add<0x112, 0xf>(v);  // row_shr:2
    v = dpp_add<0x114, 0xf>(v);  // row_shr:4
    v = dpp_add<0x118, 0xf>(v);  // row_shr:8
    v = dpp_add<0x142, 0xa>(v);  // row_bcast:15 into rows 1, 3
    v = dpp_add<0x143, 0xc>(v);  // row_bcast:31 into rows 2, 3
    return v;
}
__device__ __forceinline__ float lane_value(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Read one word of every 64-byte line of a kernel's argument block at entry,
// all in one batch.  The compiler otherwise loads the fields it needs in
// several dependent groups as the code reaches them, and each group waits a
// memory round trip for lines no cache holds yet; after this, those loads hit
// the scalar cache.
template <typename P>
__device__ __forceinline__ void touch_args(const P& p) {
    const uint32_t* w = reinterpret_cast<const uint32_t*>(&p);
    uint32_t x = 0;
#pragma unroll
    for (int i = 0; i < (int)(sizeof(P) / 4); i += 16) x ^= w[i];
    asm volatile("" ::"s"(x));
}

// Raw v_exp_f32: every argument here is <= 0, results below 2^-126 flush to 0.
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// softplus(z) = max(z, 0) + log(1 + e^{-|z|}) from the hardware exp2 / log2.
// Below v = e^{-|z|} = 1/64, where 1 + v would drop v's low bits, log(1 + v)
// is its alternating series to v^4 (relative error under v^4 / 5 < 1e-8).
__device__ __forceinline__ float softplus(float z) {
    constexpr float kLn2 = 0.69314718055994531f;
    const float v = fexp2(-fabsf(z) * kLog2e);
    const float series = v * (1.f - v * (0.5f - v * (1.f / 3.f - v * 0.25f)));
    const float direct = __builtin_amdgcn_logf(1.f + v) * kLn2;
    return fmaxf(z, 0.f) + (v < 0.015625f ? series : direct);
}

// LDS tiles are column-blocked: 16-column blocks of 64 token rows, block b
// at element offset b * 1024 (2 KB for bf16, 4 KB for fp32).  Within a block
// row r is stored at row r ^ (4 * bit3(r)) and its 16-byte units are XORed
// with bit3(r).  With that, every LDS read pattern used here touches distinct
// banks: 16 consecutive rows of one unit (C B^T operands), and 4-row groups
// 8 rows apart of the transposing reads; and the offset of block b is a
// constant, so the fragments of all blocks share one address register.
template <typename T>
__device__ __forceinline__ int boff(int r, int blk, int ec) {
    constexpr int EPU = 16 / sizeof(T);  // elements per 16-byte unit
    const int b3 = (r >> 3) & 1;
    const int pr = r ^ (b3 << 2);
    const int u = (ec / EPU) ^ b3;
    return blk * (kChunk * 16) + pr * 16 + u * EPU + ec % EPU;
}

// Issue the direct global -> LDS loads (global_load_lds_dwordx4) of
// instructions first + k*STEP (k < NI) of a column-blocked tile: instruction
// i fills the 1 KB at i KB, lane l its 16 bytes at l*16.  Tile row r is the
// global row at row0 + r * rstride (elements; negative for an anti-causal
// pass), column c at row + c.  Rows at or past clen read row 0 and columns at
// or past ccols read column 0: such entries only ever meet zero weights or
// are never read.  The per-lane offsets do not depend on the chunk, so the
// compiler keeps them out of the chunk loop; a full chunk needs no clamp.
template <int NI, int STEP, int NINST, typename T>
__device__ __forceinline__ void issue_tile(T* __restrict__ tile, const T* row0, int rstride,
                                           int first, int clen, int ccols, int lane) {
    constexpr int EPU = 16 / sizeof(T), W = 16 / EPU;  // units per block row
    const bool full = clen == kChunk;
#pragma unroll
    for (int k = 0; k < NI; ++k) {
        const int i = first + k * STEP;
        if (NINST % STEP != 0 && i >= NINST) break;
        const int j = (i % W) * 64 + lane;   // unit within the block
        const int pr = j / W, pu = j % W;    // stored row and unit
        const int b3 = (pr >> 3) & 1;
        const int r = pr ^ (b3 << 2);        // logical row
        int col = (i / W) * 16 + (pu ^ b3) * EPU;
        if (col >= ccols) col = 0;
        const int off = r * rstride + col;
        const T* g = row0 + (full || r < clen ? off : col);
        __builtin_amdgcn_global_load_lds((const void*)g,
                                         (__attribute__((address_space(3))) void*)(tile + i * 64 * EPU),
                                         16, 0, 0);
    }
}

// Wait until at most NOUT vector-memory operations of this wave are in
// flight (they retire in issue order).  A compiler builtin, so the compiler
// knows about the wait and does not repeat it.
template <int NOUT>
__device__ __forceinline__ void vm_wait() {
    static_assert(NOUT >= 0 && NOUT < 64, "vm_wait");
    // vmcnt in bits 3:0 and 15:14; expcnt (6:4) and lgkmcnt (11:8) at their maxima
    __builtin_amdgcn_s_waitcnt((NOUT & 15) | ((NOUT >> 4) << 14) | 0x0F70);
}
// Workgroup barrier after this wave's own LDS operations have completed; the
// "memory" clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void block_sync() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// 4 consecutive elements (8 or 16 bytes) at (row r, block blk, column ec) of
// a column-blocked tile; ec a multiple of 4.
template <typename T>
__device__ __forceinline__ typename Vec<T>::x4 tld4(const T* t, int r, int blk, int ec) {
    return ld4(t + boff<T>(r, blk, ec));
}

// Token-contracted MFMA fragment of block blk of a column-blocked tile: lane
// (l16, g) gets column 16*blk + l16 at tokens r0..r0+3 (slots 0-3) and
// r1..r1+3 (slots 4-7); r0, r1 are the same for the 16 lanes of a group.
// bf16 uses the gfx950 transposing read (ds_read_b64_tr_b16): lane i of a
// 16-lane group receives, in slot k, element i%4 of the 8 bytes addressed by
// lane 4k + i/4 of the group, so lane j addresses row r + j/4, columns
// 4*(j%4) .. +3 of the block.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x4 ldtr(const bf16* p) {
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(p));
    return __builtin_bit_cast(bf16x4, v);
}
__device__ __forceinline__ bf16x8 tok_frag(const bf16* t, int r0, int r1, int blk, int lane) {
    const int j = lane & 15, dr = j >> 2, ec = 4 * (j & 3);
    return cat<bf16x8, bf16x4>(ldtr(t + boff<bf16>(r0 + dr, blk, ec)),
                               ldtr(t + boff<bf16>(r1 + dr, blk, ec)));
}
__device__ __forceinline__ f32x8 tok_frag(const float* t, int r0, int r1, int blk, int lane) {
    const int ec = lane & 15;
    f32x8 v;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        v[k] = t[boff<float>(r0 + k, blk, ec)];
        v[4 + k] = t[boff<float>(r1 + k, blk, ec)];
    }
    return v;
}

// Operand fragment over the state dimension (K = n) of tile row r for the K
// step kk: a lane of group g holds n = 32kk + 4g + (0..3) in slots 0-3 and
// n = 32kk + 16 + 4g + (0..3) in slots 4-7 (zeros past N).  This is the K
// order of a pair of state result tiles (rows 4g..4g+3 of blocks 2kk and
// 2kk+1), so the state feeds H^T C^T with no data movement.
template <int N, typename T>
__device__ __forceinline__ typename Vec<T>::x8 tile_frag(const T* tile, int r, int kk, int g) {
    using X4 = typename Vec<T>::x4;
    // the hi half sits exactly one column block after the lo half, written
    // as such so that both come from one base address (one paired read into
    // the fragment's own registers)
    const T* const plo = tile + boff<T>(r, 2 * kk, 4 * g);
    const X4 lo = ld4(plo);
    X4 hi = {};
    if (N % 32 == 0 || 2 * kk + 1 < N / 16) hi = ld4(plo + kChunk * 16);
    return cat<typename Vec<T>::x8, X4>(lo, hi);
}

// Per-head, per-chunk decay factors (cs = within-chunk cumulative -d in log2
// units, c_k = cs at the last token of 16-token block k-1, c_0 = 0).  For s in
// block sb < tb and t in block tb,
//   e^{cs_t - cs_s} d_s = fa_s * fm(tb, sb) * fb_t,
//   fa_s = 2^{c_{sb+1} - cs_s} d_s,  fm = 2^{c_tb - c_{sb+1}},  fb_t = 2^{cs_t - c_tb},
// each factor <= 1, so off-diagonal mask tiles need no exponentials.
struct __attribute__((aligned(16))) Decay {  // read with 16-byte vector loads
    float cs2[kChunk];  // cs
    float dt[kChunk];   // d_s (0 past the end of the sequence)
    float w[kChunk];    // 2^{cs_last - cs_s} d_s   (state update weights)
    float fa[kChunk];
    float fb[kChunk];
    float fe[kChunk];   // 2^{cs_t}
    float fm[8];        // block pairs (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
};

// The factors a chunk-state pass needs (a quarter of Decay's LDS): the
// cumulative log-decay and the state update weights -- 2^{cs_last - cs_s} d_s,
// or 2^{cs_s} (0 past the end) for the output-gradient states.
struct __attribute__((aligned(16))) DecayS {
    float cs2[kChunk];
    float w[kChunk];
};
// Both directions' chunk-state factors (the pass forming the forward and the
// reverse span states in one walk): the forward weights as in DecayS, and
// wr = 2^{cs_{s-1}} d_s, the decay of the chunk's tokens before s times d_s.
struct __attribute__((aligned(16))) DecayS2 {
    float cs2[kChunk];
    float w[kChunk];
    float wr[kChunk];
};
__device__ __forceinline__ float chunk_decay(const Decay& D) { return D.fe[kChunk - 1]; }
__device__ __forceinline__ float chunk_decay(const DecayS& D) { return fexp2(D.cs2[kChunk - 1]); }
__device__ __forceinline__ float chunk_decay(const DecayS2& D) { return fexp2(D.cs2[kChunk - 1]); }

// Span states are kept in MFMA result order so each wave moves 64 contiguous
// 4-value groups: within one (span, head) block of P*N values, state entry
// (n, p) with p = 16*pb + l, n = 16*nb + 4*g + i sits at
// ((pb*NB + nb)*64 + 16*g + l)*4 + i.
__device__ __forceinline__ int64_t state_off(int pb, int nb, int lane, int NB) {
    return ((int64_t)(pb * NB + nb) * 64 + lane) * 4;
}

// One wave forms a head's decay factors for one chunk from d_raw as loaded
// into LDS (a bf16 value sits in the low half of its 32-bit slot).
template <typename T>
__device__ __forceinline__ void decay_factors(Decay& D, uint32_t raw, float d_init, int clen,
                                              int lane) {
    const float draw = __uint_as_float(sizeof(T) == 2 ? raw << 16 : raw);
    const float dt = lane < clen ? softplus(draw + d_init) : 0.f;
    const float v = wave_prefix_sum(-dt * kLog2e);
    const float c1 = lane_value(v, 15), c2 = lane_value(v, 31);
    const float c3 = lane_value(v, 47), c4 = lane_value(v, 63);
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
template <typename T>
__device__ __forceinline__ void decay_factors(DecayS& D, uint32_t raw, float d_init, int clen,
                                              int lane, bool grad) {
    const float draw = __uint_as_float(sizeof(T) == 2 ? raw << 16 : raw);
    const float dt = lane < clen ? softplus(draw + d_init) : 0.f;
    const float v = wave_prefix_sum(-dt * kLog2e);
    D.cs2[lane] = v;
    D.w[lane] = grad ? (lane < clen ? fexp2(v) : 0.f) : fexp2(lane_value(v, 63) - v) * dt;
}
template <typename T>
__device__ __forceinline__ void decay_factors(DecayS2& D, uint32_t raw, float d_init, int clen,
                                              int lane, bool) {
    const float draw = __uint_as_float(sizeof(T) == 2 ? raw << 16 : raw);
    const float dt = lane < clen ? softplus(draw + d_init) : 0.f;
    const float v = wave_prefix_sum(-dt * kLog2e);
    D.cs2[lane] = v;
    D.w[lane] = fexp2(lane_value(v, 63) - v) * dt;
    D.wr[lane] = fexp2(v + dt * kLog2e) * dt;  // v + dt log2e: the sum over tokens before s
}

}  // namespace
}  // namespace ssd
