/*
 * libssd -- Mamba-2 SSD selective state-space scan, forward and backward, on one
 * MI355X (gfx950).  C ABI: plain pointers and sizes, no C++ types, no
 * exceptions across the boundary.
 *
 * What it computes ("Mamba-2架构与LaCT并行计算技术解析", §1.1 state update):
 * for every sequence and head, in processing order t,
 *     d_t = softplus(d_raw_t + d_init)
 *     H_t = exp(-d_t) * H_{t-1} + d_t * B_t^T X_t        (H: d_state x headdim)
 *     y_t = C_t H_t
 * with independent heads (§1.2 of the same page), H_{-1} = init_state (zeros
 * when NULL), and final_state = H after the sequence's last processed token.
 * The scan is evaluated in the chunked semiseparable form of
 * "长序列 Mamba 多卡训练，算力和显存怎么同时省", §一 (a dense diagonal block per
 * chunk plus a small state handed between chunks), with the state handed on
 * as (decay, state) pairs as in the Mamba context-parallel scheme of
 * "揭秘MindSpeed-LLM多潜在注意力（MLA）与Mamba上下文并行实现原理", §三.2.
 *
 * Packed variable-length batches (cu_seqlens) follow §三 of the qwbw.cn page
 * above: each segment [cu[i], cu[i+1]) is an independent sequence whose
 * state starts from init_state[i].  reverse != 0 runs every sequence from
 * its last token to its first (the flipped pass of the bidirectional mode,
 * jsqmd.com page §3.1) and writes y at each token's own position, so no
 * flipped copy of any tensor is made.
 *
 * Ownership: the caller owns every buffer.  The library allocates no device
 * memory, does not synchronize the stream (except ssd_fwd / ssd_bwd with
 * SSD_CHECK=1 in the environment, which copy cu_seqlens to the host to
 * check it), and keeps no mutable global state; calls on different streams
 * with separate workspaces may run concurrently.  All argument checks run
 * on the host before any launch; on an error status nothing is launched and
 * no output is written.  The library reads one environment variable,
 * SSD_CHECK; its tuning choices are explicit arguments (ssd_tuning).  (The
 * one exception to "no global state" is ssd_fwd_noalloc's per-device
 * scratch array and the address it caches for each device.)
 */
#ifndef LIBSSD_SSD_H
#define LIBSSD_SSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSD_ABI_VERSION 8

/* Status codes: 0 is success, every error is negative. */
enum {
    SSD_OK = 0,
    SSD_ERR_NULL_ARG = -1,        /* a required pointer is NULL                 */
    SSD_ERR_SHAPE = -2,           /* inconsistent or out-of-range sizes,
                                     strides or tuning values                  */
    SSD_ERR_DTYPE = -3,           /* unknown dtype code                          */
    SSD_ERR_ALIGN = -4,           /* pointer or stride misaligned (16 bytes;
                                     d_raw / dd_raw: their element size)       */
    SSD_ERR_UNSUPPORTED = -5,     /* valid but not built (chunk_size, d_state..) */
    SSD_ERR_WORKSPACE = -6,       /* workspace NULL or smaller than required     */
    SSD_ERR_HIP = -7,             /* a HIP launch or runtime call failed         */
    SSD_ERR_CU_SEQLENS = -8,      /* cu_seqlens invalid (checked only when the
                                     environment sets SSD_CHECK=1)               */
    SSD_ERR_OVERLAP = -9,         /* init_state and final_state (or d_final and
                                     dinit_state) overlap without being the
                                     same buffer                                */
    SSD_ERR_SCRATCH = -10         /* ssd_fwd_noalloc: the sizes need more
                                     scratch than its fixed buffer holds       */
};

/* Element type of x, d_raw, B, C and y.  States are always float32. */
enum { SSD_F32 = 0, SSD_BF16 = 1 };

/* Problem sizes.  Tokens are laid out [batch][seqlen]; with cu_seqlens the
 * batch must be 1 and seqlen is the total packed length. */
typedef struct ssd_dims {
    int32_t batch;       /* b >= 1                                             */
    int64_t seqlen;      /* L >= 0 tokens per batch row                        */
    int32_t nheads;      /* H >= 1                                             */
    int32_t headdim;     /* P: multiple of 16, 16..512                         */
    int32_t d_state;     /* N: 16, 32, 64, 128 or 256 (bf16); up to 128 (f32) */
    int32_t ngroups;     /* G >= 1, divides H; head h reads group h*G/H        */
    int32_t chunk_size;  /* must be 64                                         */
    int32_t nseq;        /* number of cu_seqlens segments (0 without them)     */
    int32_t dtype;       /* SSD_F32 or SSD_BF16                                */
} ssd_dims;

/*
 * Element strides of the per-token tensors.  Token index k = bi * L + l
 * runs over the flattened [b, L] tokens (so a batch row is L token strides
 * further on); the innermost dimension is always contiguous.  Element
 * (k, h, p) of x is at x + k * x_token + h * x_head + p, element (k, g, n)
 * of B at B + k * B_token + g * B_group + n, and so on.  They let x, B, C
 * and d_raw be views of one projection output, as in "Mamba-2架构与LaCT
 * 并行计算技术解析" §1.1, where X, B, C and the raw step come from one
 * linear map of the input.  Rules (checked on the host, SSD_ERR_ALIGN /
 * SSD_ERR_SHAPE): every stride is >= 0 and at most 2^24; the strides of x,
 * B, C, y and dy are multiples of 16 bytes; d_raw's are any element count.
 * A NULL layout means every tensor is contiguous: x_token = H*P, x_head =
 * P, d_raw_token = H, d_raw_head = 1, B_token = C_token = G*N, B_group =
 * C_group = N, y and dy like x.
 */
typedef struct ssd_layout {
    int64_t x_token, x_head;         /* x  [b, L, H, P]                       */
    int64_t d_raw_token, d_raw_head; /* d_raw [b, L, H]                       */
    int64_t B_token, B_group;        /* B  [b, L, G, N]                       */
    int64_t C_token, C_group;        /* C  [b, L, G, N]                       */
    int64_t y_token, y_head;         /* y  [b, L, H, P] (ssd_fwd's output,
                                        ssd_bwd's input)                      */
    int64_t dy_token, dy_head;       /* dy [b, L, H, P] (ssd_bwd only)        */
} ssd_layout;

/*
 * Explicit choices that override the planner (timing sweeps and tests; the
 * library reads no tuning from the environment).  Zero in every field means
 * the planner's choice, so a zero-filled struct equals passing NULL.
 * Values the sizes cannot take return SSD_ERR_SHAPE (SSD_ERR_UNSUPPORTED for
 * shapes that are not built).
 */
typedef struct ssd_tuning {
    int32_t kernel;           /* 1: span kernels; 2: head-wave kernels (bf16,
                                 d_state 64 or 128)                           */
    int32_t chunks_per_span;  /* 1..64 chunks walked by one workgroup         */
    int32_t state_pass;       /* batch mode, span kernels: 1 state_pass launch
                                 (plan 0); 2 folded into the scan (plan 1);
                                 3 one fused launch (plan 2)                  */
    int32_t heads_state;      /* heads per state workgroup: 1, 2 (head-wave: 4)*/
    int32_t heads_scan;       /* heads per scan workgroup: 1, 2 (head-wave: 4) */
    int32_t cols_per_wave;    /* head-wave kernels: 32, or 64 at d_state 64    */
    int32_t bwd_heads;        /* heads per backward gradient workgroup        */
    int32_t bwd_state_chunks; /* chunks per backward chunk-state workgroup: 1, 4 */
    int32_t state_f32;        /* 1: span states stored in float32 for bf16
                                 inputs (span kernels, plans 0 and 1)        */
    int32_t reserved[7];      /* must be 0                                    */
} ssd_tuning;

/* ABI version of the loaded library (SSD_ABI_VERSION it was built with). */
int ssd_abi_version(void);

/* Bytes of device workspace ssd_fwd needs for these sizes with the
 * planner's choices (0 when the sizes are invalid).  A pure function of
 * *dims: never of data or the environment. */
size_t ssd_fwd_workspace_bytes(const ssd_dims* dims);

/*
 * Forward scan.  Device pointers:
 *   x           [b, L, H, P]   dtype
 *   d_raw       [b, L, H]      dtype
 *   d_init      scalar added to d_raw before softplus
 *   B, C        [b, L, G, N]   dtype
 *   init_state  [S, H, N, P]   float32 contiguous, or NULL for zeros
 *   cu_seqlens  [nseq + 1]     int32 on the device, or NULL; must start at 0,
 *               be non-decreasing and end at L (only checked when SSD_CHECK=1;
 *               other values are clamped into range so no access leaves the
 *               buffers, but the result is then unspecified)
 *   reverse     0 = causal, 1 = anti-causal within each sequence
 *   y           output [b, L, H, P] of dtype
 *   final_state output [S, H, N, P] float32 contiguous, or NULL to skip; it
 *               may be the same buffer as init_state (an in-place state
 *               update between calls), but not overlap it otherwise
 *               (SSD_ERR_OVERLAP)
 *   layout      strides of x, d_raw, B, C and y (see ssd_layout), or NULL
 *   workspace   device scratch of at least ssd_fwd_workspace_bytes(dims)
 *               bytes, 256-byte aligned.  It needs no initialization and
 *               holds nothing the caller reads; calls that overlap in time
 *               need separate workspaces.  Its first 256 bytes are a header
 *               of 32-bit words: word 2 counts the bounded flag waits of the
 *               last fused launch that ran out (it stays 0).
 *   stream      hipStream_t to launch on (NULL = default stream)
 * S is b without cu_seqlens and nseq with them.  x, B, C and y must be
 * 16-byte aligned, d_raw aligned to its element size; they may be NULL only
 * when b*L == 0.  y must not overlap the inputs.  Returns SSD_OK once the
 * work is queued on the stream.
 */
int ssd_fwd(const ssd_dims* dims, const ssd_layout* layout,
            const void* x, const void* d_raw, float d_init,
            const void* B, const void* C,
            const float* init_state, const int32_t* cu_seqlens, int32_t reverse,
            void* y, float* final_state,
            void* workspace, size_t workspace_bytes,
            void* stream);

/* How ssd_fwd / ssd_bwd split a problem of these sizes (a pure function of
 * *dims and *tuning). */
typedef struct ssd_plan_info {
    int32_t chunks_per_span;   /* 64-token chunks walked by one workgroup; the
                                  state stays on chip inside a span          */
    int32_t col_groups;        /* headdim columns are split in groups of 64  */
    int64_t nspan;             /* span slots (upper bound with cu_seqlens)   */
    uint64_t workspace_bytes;  /* workspace ssd_fwd_ex needs with this tuning
                                  (= ssd_fwd_workspace_bytes(dims) for NULL) */
    int32_t fused_pass;        /* 0: stages STATE, PASS and SCAN launch one
                                  kernel each.  1: SCAN forms every span's
                                  incoming state from the span states itself
                                  and PASS launches nothing.  2: SCAN is one
                                  launch that does STATE, PASS and SCAN
                                  (their workgroups hand span states to each
                                  other); STATE and PASS launch nothing.
                                  The planner takes 1 in batch mode with
                                  1..8 spans per sequence, else 0; always 0
                                  with head-wave kernels, and whenever
                                  final_state is init_state.               */
    int32_t head_wave;         /* 1: head-wave kernels (one wave computes every
                                  product of one head for cols_per_wave
                                  headdim columns); 0: span kernels (four
                                  waves per head, 16 columns each)          */
    int32_t heads_per_wg;      /* heads sharing one scan workgroup's B / C
                                  tiles                                     */
    int32_t cols_per_wave;     /* headdim columns one wave computes          */
    int32_t heads_per_state_wg;/* heads of one state workgroup               */
    int32_t state_bytes;       /* bytes of one stored span-state entry       */
    uint64_t bwd_workspace_bytes; /* workspace ssd_bwd_ex needs (0: the
                                  backward is not built for these sizes)     */
    int32_t bwd_heads_per_wg;  /* heads of one backward gradient workgroup   */
    int32_t bwd_head_subsets;  /* dB / dC partials added after it            */
    int32_t bwd_state_chunks;  /* chunks of one backward chunk-state workgroup */
    int32_t reserved;
} ssd_plan_info;

/* Fills *out for these sizes and tuning (NULL = the planner's choices);
 * returns the status ssd_fwd_ex's size and tuning checks would give. */
int ssd_fwd_plan(const ssd_dims* dims, const ssd_tuning* tuning, ssd_plan_info* out);

/* Stages of ssd_fwd, one kernel launch each, in this order. */
enum {
    SSD_STAGE_TABLE = 1,  /* span table from cu_seqlens (no-op without them) */
    SSD_STAGE_STATE = 2,  /* per-span local states and decays (folded into
                             SSD_STAGE_SCAN when fused_pass is 2)           */
    SSD_STAGE_PASS = 4,   /* state passing across spans, final_state (folded
                             into SSD_STAGE_SCAN when fused_pass is 1 or 2) */
    SSD_STAGE_SCAN = 8,   /* per-chunk outputs y                            */
    SSD_STAGE_ALL = 15
};

/* ssd_fwd with explicit tuning (NULL = the planner's choices; the workspace
 * is then ssd_fwd_plan's workspace_bytes for that tuning) and restricted to
 * the stages in stage_mask, for callers that time or interleave work
 * between stages.  Running the stages in the order above on one stream with
 * one workspace (left untouched in between) and the same tuning gives
 * exactly ssd_fwd_ex's result with SSD_STAGE_ALL.
 *
 * Between stages the workspace can be read (span kernels, fused_pass 0 or
 * 1; for inspection and tests).  After SSD_STAGE_STATE, bytes from 256 hold
 * nspan x H span states of P x N entries, state_bytes each (span s = sequence
 * x spans per sequence + span within it; spans run from the end of a sequence
 * when reverse is set): the state of the span's tokens from a zero state,
 * entry (n, p) at ((p / 16 * N/16 + n / 16) * 64 + lane) * 4 + i with lane =
 * 16 (n % 16 / 4) + p % 16, i = n % 4.  The nspan x H float32 decay products
 * exp(-sum of d over the span) follow at the next 256-byte boundary.  After
 * SSD_STAGE_PASS (fused_pass 0) each state slot holds the state entering its
 * span instead. */
int ssd_fwd_ex(uint32_t stage_mask, const ssd_dims* dims, const ssd_tuning* tuning,
               const ssd_layout* layout,
               const void* x, const void* d_raw, float d_init,
               const void* B, const void* C,
               const float* init_state, const int32_t* cu_seqlens, int32_t reverse,
               void* y, float* final_state,
               void* workspace, size_t workspace_bytes,
               void* stream);

/*
 * Both directions of the bidirectional mode (jsqmd.com page §3.1: the
 * causal scan and the same scan over the time-flipped sequence, their
 * outputs concatenated) in one call, batch mode only (nseq > 0 returns
 * SSD_ERR_SHAPE):
 * y_fwd, final_fwd are ssd_fwd's outputs with reverse = 0 from init_fwd,
 * y_rev, final_rev those with reverse = 1 from init_rev.  Both outputs
 * follow layout's y strides (for example the two halves of one
 * [b, L, H, 2P] tensor).  Arguments and checks otherwise as ssd_fwd_ex
 * with every stage; either direction's error is returned before anything
 * is queued.  Where every span of a sequence is whole (L a multiple of
 * 64 times ssd_fwd_plan's chunks_per_span) and the plan keeps a separate
 * state stage (fused_pass 0 or 1), the span states of both directions are
 * formed in one pass over x, B and d_raw; otherwise the two directions run
 * as two ssd_fwd_ex calls.  Each output agrees with the one-direction
 * call's to rounding (the states are accumulated in another order).
 *   workspace   at least ssd_fwd_bidir_workspace_bytes(dims) bytes (two
 *               forward workspaces), 256-byte aligned, no initialization
 */
size_t ssd_fwd_bidir_workspace_bytes(const ssd_dims* dims);

int ssd_fwd_bidir(const ssd_dims* dims, const ssd_tuning* tuning, const ssd_layout* layout,
                  const void* x, const void* d_raw, float d_init,
                  const void* B, const void* C,
                  const float* init_fwd, const float* init_rev,
                  void* y_fwd, void* y_rev, float* final_fwd, float* final_rev,
                  void* workspace, size_t workspace_bytes,
                  void* stream);

/*
 * Backward pass: the gradients of a loss L with respect to every input of
 * ssd_fwd, given dL/dy and dL/d final_state.  The pages name this pass (the
 * Mamba context-parallel backward of "揭秘MindSpeed-LLM多潜在注意力（MLA）与Mamba
 * 上下文并行实现原理", §三.2) without writing it out; it is the derivative of
 * the map defined above:
 *   G_t = C_t^T dy_t + exp(-d_{t+1}) G_{t+1}   (G = dL/dH; G_T adds d_final)
 *   dx_t = d_t B_t G_t,   dB_t = d_t G_t x_t^T,   dC_t = H_t dy_t,
 *   dd_t = < G_t, -exp(-d_t) H_{t-1} + B_t^T x_t >,
 *   d_raw gradient dd_t * sigmoid(d_raw_t + d_init), d_init gradient its sum,
 *   init_state gradient exp(-d_0) G_0,
 * with dB and dC summed over the heads of each group.  It runs in the same
 * chunked form as ssd_fwd (states entering every chunk, then per-chunk
 * gradients), all in the processing order given by reverse.
 *
 * Built for d_state 16, 32, 64 or 128 (bf16) or 16, 32 (float32); other
 * d_state values return SSD_ERR_UNSUPPORTED.  Any headdim ssd_fwd accepts.
 *
 * Arguments as ssd_fwd, plus:
 *   y           not read (the gradients are formed from the inputs and the
 *               chunk states); may be NULL.  layout->y_* is not checked.
 *   dy          dL/dy, dtype, strides layout->dy_*
 *   d_final     dL/d final_state [S, H, N, P] float32, or NULL for zeros
 *   dx          output, dtype, laid out like x (strides layout->x_*)
 *   dd_raw      output, dtype, laid out like d_raw
 *   dB, dC      outputs, dtype, laid out like B and C
 *   dinit_state output [S, H, N, P] float32 (the gradient at the given
 *               init_state, or at zeros when it is NULL), or NULL to skip;
 *               it may be the same buffer as d_final, but not overlap it
 *               otherwise (SSD_ERR_OVERLAP)
 *   dd_init     output: one float32 on the device, or NULL to skip
 *   workspace   at least ssd_bwd_workspace_bytes(dims) bytes, 256-byte
 *               aligned, no initialization needed; calls that overlap in
 *               time need separate workspaces
 * x, B, C, dy, dx, dB and dC must be 16-byte aligned.  The gradients must
 * not overlap the inputs.  Outputs for tokens outside every cu_seqlens
 * segment are not written.  Returns SSD_OK once the work is queued.
 */
size_t ssd_bwd_workspace_bytes(const ssd_dims* dims);

int ssd_bwd(const ssd_dims* dims, const ssd_layout* layout,
            const void* x, const void* d_raw, float d_init,
            const void* B, const void* C,
            const float* init_state, const int32_t* cu_seqlens, int32_t reverse,
            const void* y, const void* dy, const float* d_final,
            void* dx, void* dd_raw, void* dB, void* dC,
            float* dinit_state, float* dd_init,
            void* workspace, size_t workspace_bytes,
            void* stream);

/* ssd_bwd with explicit tuning (NULL = the planner's choices; the workspace
 * is then ssd_fwd_plan's bwd_workspace_bytes for that tuning). */
int ssd_bwd_ex(const ssd_dims* dims, const ssd_tuning* tuning, const ssd_layout* layout,
               const void* x, const void* d_raw, float d_init,
               const void* B, const void* C,
               const float* init_state, const int32_t* cu_seqlens, int32_t reverse,
               const void* y, const void* dy, const float* d_final,
               void* dx, void* dd_raw, void* dB, void* dC,
               float* dinit_state, float* dd_init,
               void* workspace, size_t workspace_bytes,
               void* stream);

/*
 * ssd_fwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation):
 * the same scan with the planner's choices, its scratch taken from a fixed
 * array inside the library instead of a workspace argument.  Each GPU the
 * library runs on holds one such array of ssd_fwd_noalloc_max_bytes()
 * bytes (64 MiB) until the process ends; its device address is looked up
 * once per device, on the first call with that device current.  The call
 * allocates nothing and synchronizes nothing (SSD_CHECK=1 aside).
 * Arguments as ssd_fwd without the workspace.  Sizes whose workspace
 * (ssd_fwd_workspace_bytes) exceeds the array return SSD_ERR_SCRATCH before
 * any HIP call.  Every call on one GPU uses that GPU's one array: calls
 * that overlap in time on one GPU (different streams, or threads) race and
 * give unspecified results; nothing in the array needs to start at zero.
 */
int ssd_fwd_noalloc(const ssd_dims* dims, const ssd_layout* layout,
                    const void* x, const void* d_raw, float d_init,
                    const void* B, const void* C,
                    const float* init_state, const int32_t* cu_seqlens, int32_t reverse,
                    void* y, float* final_state,
                    void* stream);

/* Bytes of ssd_fwd_noalloc's fixed scratch array on each GPU. */
size_t ssd_fwd_noalloc_max_bytes(void);

/* Static description of a status code (never NULL). */
const char* ssd_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* LIBSSD_SSD_H */
