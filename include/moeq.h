/* moeq.h — C ABI of the routed Mixture-of-Experts feed-forward layer over
 * block-quantised expert weights, for AMD Instinct MI355X (gfx950).
 *
 * The layer (what the pages describe, restated):
 *   - the router gives every token one logit per expert and keeps k experts with
 *     normalised weights ("Nebula" page, "How it works"; "How Neural runs a
 *     120-billion-parameter model on one gaming PC", section "How one token and
 *     one prompt are processed": the router emits expert ids and weights);
 *   - the device sorts the (token, expert) pairs into per-expert groups and
 *     streams each selected expert's weights once for all of its tokens, finding
 *     them through a table of expert addresses held in device memory (NInfer
 *     Qwen3.8-Flash-Next page, MoE execution notes; Neural page, "Prompt
 *     processing");
 *   - each expert applies a fused gate/up projection, SwiGLU and a down
 *     projection, and the gate-weighted expert outputs are summed per token in a
 *     fixed order (NInfer page, MoE execution notes: the sum is independent of
 *     which expert completes first), plus an optional always-on shared expert
 *     ("Running Qwen3.8-Flash-Next on a 32 GB Mac with Transformers",
 *     "Architecture").
 *
 * Formulas (notation: T tokens, H hidden, I intermediate, E experts, top-k):
 *   l[t,e]  = sum_h x[t,h] * router_w[e,h] + router_b[e]
 *   ids[t]  = the k experts with the largest l[t,.], ordered by (-l, e): ties go
 *             to the lower expert index
 *   g[t,j]  = exp(l[t,ids[t,j]] - l[t,ids[t,0]]) / sum_j' exp(...)
 *   pair p  = t*k + j (routed) or T*k + t (shared expert, bucket E)
 *   h_p[i]  = silu(Wg_e[i,:] . x[t]) * (Wu_e[i,:] . x[t]),  silu(a) = a/(1+e^-a)
 *   o_p[n]  = Wd_e[n,:] . h_p
 *   y[t]    = sum_j g[t,j] * o_(t*k+j) + s_t * o_(T*k+t)   (j ascending, shared last)
 *   s_t     = 1, or sigmoid(shared_gate_w . x[t]) when shared_gate_w != NULL
 *
 * Packed matrix [N rows][K cols] (N a multiple of 16, K a multiple of 32), blocks of
 * 32 consecutive values along a row, nkb = K/32 blocks per row.  Within a block, code
 * byte j holds element 2j in its low nibble and element 2j+1 in its high nibble.
 * The matrix is a code plane followed by a scale plane, both stored tile-major: rows
 * form tiles of 16 (tile t = rows 16t .. 16t+15, row m = row % 16) and a row's blocks
 * form steps of 4 (step s = blocks 4s .. 4s+3; the last step holds r = nkb - 4s < 4
 * blocks when nkb % 4 != 0; block b = 4s + g):
 *   code plane at byte 0, N*K/2 bytes: the 16 code bytes of block (row 16t+m, 4s+g)
 *     start at byte t*8*K + 1024*s + (16*g + m)*16, so one tile's step is one
 *     contiguous run of 256*r bytes;
 *   scale plane at byte S = round_up(N*K/2, 256), N*nkb scales: the scale of block
 *     (row 16t+m, 4s+g) is entry t*16*nkb + 64*s + i of the plane, where
 *       MXFP4: i = 16*g + m, entries are bytes (byte S + entry);
 *       CB4:   i = m*r + g, entries are little-endian fp16 (bytes S + 2*entry, +1);
 *   moe_packed_bytes gives S + N*nkb (MXFP4) or S + 2*N*nkb (CB4).
 *   MXFP4: code = FP4 E2M1, scale = E8M0 byte u, element = e2m1 * 2^(u-127)
 *     (OCP Microscaling v1.0; the Neural page names MXFP4 experts, "What it runs
 *     on and what it runs": 13,219,200 bytes per gpt-oss-120B expert, which this
 *     layout reproduces exactly);
 *   CB4: code = index into a 16-entry int8 codebook, scale = IEEE fp16 bits,
 *     element = fp16 * codebook[index]; 18 bytes per 32 values (NInfer page,
 *     n-gram table paragraph: 1,440 bytes for 16 rows of 160 IQ4_NL values).
 *   MXFP4_PS (the packed scale store of "How Neural runs a 120-billion-parameter model
 *     on one gaming PC", section "What it runs on and what it runs": 12,839,040 bytes per
 *     gpt-oss-120B expert, code bytes kept and scale rows re-encoded, with bit-identical
 *     outputs): the MXFP4 code plane, then at byte S the N row bases (byte S + row) and
 *     then N*nkb/2 bytes of 4-bit deltas: the delta of the block whose MXFP4 scale is
 *     entry i of the scale plane is nibble i, byte S + N + i/2, low nibble for even i.
 *     The block's E8M0 byte is base(row) + delta; everything else is MXFP4.
 *     moe_packed_bytes gives S + N + N*nkb/2.
 *   AFF3 (3-bit affine, group 64: "Running Qwen3.8-Flash-Next on a 32 GB Mac with
 *     Transformers", section "Where every weight lives": 3-bit MLX affine experts, group
 *     64, 2.15 MB per expert of its hidden-2,560 / intermediate-640 model, which this
 *     layout reproduces exactly; the bit packing is this library's): K a multiple of 128;
 *     element = fp16 scale * q + fp16 bias, q in 0..7, one (scale, bias) per 64
 *     consecutive values of a row.  Rows in tiles of 16, columns in steps of 128: the
 *     value at (row 16t+m, column 128s + 32j + 8g + i) (j < 4, g < 4, i < 8) belongs to
 *     the 12 bytes at t*6*K + 768*s + 12*(16g+m), three little-endian 32-bit words; with
 *     P = 4j + i/2 and h = i%2, for P < 15 it is bits 3*(P%5) + 16h .. +2 of word P/5, and
 *     for P = 15 bit k of q is bit 15 + 16h of word k.  At S3 = round_up(N*K*3/8, 256)
 *     follow per (t, s) 128 bytes: at 8m the fp16 scale and bias of row 16t+m for columns
 *     128s .. 128s+63, then for 128s+64 .. 128s+127.  moe_packed_bytes gives
 *     S3 + N*(K/64)*4.  The layer runs on the decode kernels only: calls of more than 32
 *     tokens run them on chunks of 32 (MOE_PATH_PREFILL and the bucketing debug outputs
 *     of such calls are refused with MOE_ERR_UNSUPPORTED); H and I must be multiples
 *     of 128 (else MOE_ERR_UNSUPPORTED).
 *   Expert e's gate_up matrix is [2I][H] (rows 0..I-1 gate, I..2I-1 up); its
 *   down matrix is [H][I].
 *
 * Conventions for every entry point:
 *   - Pointers are HIP device pointers unless marked [host].  The caller owns
 *     every buffer; the library keeps no pointer after a call returns.
 *   - Work is enqueued on `stream` and the call returns without waiting.  No
 *     call allocates memory, synchronises, or reads device memory on the host,
 *     so every call can be captured in a HIP graph.
 *   - Arguments are validated on the host before anything is enqueued; on
 *     failure a negative moe_status is returned and no output is touched.
 *     T == 0 returns MOE_OK once the layer descriptor is valid and enqueues nothing
 *     (buffers of zero size may then be NULL).
 *   - A launch failure returns MOE_ERR_HIP; faults during execution surface at
 *     the caller's next synchronisation, as with any stream API.
 *   - No C++ exception crosses the ABI and nothing is printed.  The library is
 *     reentrant: it keeps no state between calls besides the caller's workspace
 *     (and, for moe_forward_noalloc, its per-device scratch array and its address).
 *   - Calls that share a workspace must not overlap in time (same stream, or
 *     ordered by events).
 *   - No GPU block ever waits for another block: where a kernel needs results of
 *     other blocks of the same launch, each block checks once, after its own results
 *     have landed, and the block that finds them all complete does the dependent work.
 *     Results therefore do not depend on which blocks the GPU runs at the same time
 *     (other streams or processes may hold any share of the compute units).
 */
#ifndef MOEQ_H
#define MOEQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1,  /* null pointer, bad size or dtype */
  MOE_ERR_UNSUPPORTED = -2,  /* outside the supported shape range */
  MOE_ERR_ALIGNMENT = -3,    /* a buffer is not 16-byte aligned */
  MOE_ERR_WORKSPACE = -4,    /* workspace missing or smaller than moe_workspace_bytes */
  MOE_ERR_HIP = -5           /* a HIP launch failed */
} moe_status;

typedef enum { MOE_WFMT_MXFP4 = 1, MOE_WFMT_CB4 = 2, MOE_WFMT_MXFP4_PS = 3, MOE_WFMT_AFF3 = 4 } moe_wfmt;
typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Path selection for moe_forward: AUTO picks the decode kernels for small batches
 * (up to 10 tokens for MXFP4 layers and 32 for CB4 layers, where they are faster)
 * and the grouped-GEMM prefill kernels otherwise; the other two force one path
 * (both compute the same layer; DECODE accepts up to 32 tokens). */
typedef enum { MOE_PATH_AUTO = 0, MOE_PATH_DECODE = 1, MOE_PATH_PREFILL = 2 } moe_path;

/* [host] layer descriptor; read during a call only. */
typedef struct {
  int32_t hidden;              /* H: multiple of 32, 32..16384 */
  int32_t inter;               /* I: multiple of 32, 32..16384 */
  int32_t n_experts;           /* E: 1..1024 */
  int32_t top_k;               /* k: 1..min(E, 16) */
  int32_t wfmt;                /* moe_wfmt, the same for every expert */
  int32_t has_shared;          /* 1: slot E of the pointer tables is an always-on shared expert */
  const float *router_w;       /* [E][H] fp32 */
  const float *router_b;       /* [E] fp32, or NULL */
  const void *const *gate_up;  /* device array of E+has_shared device pointers -> packed [2I][H] */
  const void *const *down;     /* device array of E+has_shared device pointers -> packed [H][I] */
  const int8_t *codebook;      /* CB4: [16] int8; every other format: must be NULL */
  const float *shared_gate_w;  /* [H] fp32, or NULL (shared weight 1); ignored without a shared expert */
  float omit_below;            /* marginal-expert omission threshold tau in [0, 1]; 0: off (below) */
} moe_layer;

/* Marginal-expert omission ("Nebula" page, "Benchmark results": experts under a
 * 10% gate are dropped as marginal; the renormalisation is this library's reading).  With
 * omit_below = tau > 0, after the top-k softmax a routed pair j > 0 whose gate
 * g[t,j] < tau (compared in fp64) is omitted: it reports expert id -1 and weight 0, is in
 * no bucket and contributes nothing; the kept gates are renormalised to sum to 1,
 * g'[t,j] = exp(l_j - l_0) / sum over kept j' of exp(l_j' - l_0).  The first (largest)
 * pair is always kept; the shared expert is never omitted.  tau = 0 changes nothing. */

/* [host] Bytes of one packed matrix [rows][cols] in the layout above; 0 if cols is not
 * a positive multiple of 32 (of 128 for AFF3), rows is not a positive multiple of 16, or
 * the format is unknown. */
size_t moe_packed_bytes(int32_t wfmt, int32_t rows, int32_t cols);

/* [host] Workspace bytes moe_forward / moe_router_topk / moe_bucket need for up
 * to T_max tokens (0 if the descriptor is invalid).  The workspace is scratch
 * except for its first 18432 bytes, which hold synchronisation words: they must be
 * zero before the workspace's first use (e.g. hipMemset once after allocation),
 * and every completed call leaves them zero.  Everything past them is rewritten
 * by every call. */
size_t moe_workspace_bytes(const moe_layer *L, int32_t T_max);

/* Router logits, top-k and softmax gates for T tokens of x ([T][H], dtype
 * x_dtype).  Writes topk_ids [T][k] int32 and topk_w [T][k] fp32 (with omission:
 * id -1 and weight 0 for an omitted pair). */
int moe_router_topk(const moe_layer *L, const void *x, int32_t x_dtype, int32_t T,
                    int32_t *topk_ids, float *topk_w, void *ws, size_t ws_bytes,
                    void *stream);

/* Stable counting sort of the pairs p = t*k + j by expert (increasing p inside
 * a bucket); with a shared expert, pairs T*k + t form bucket E.
 * counts [E+1], offsets [E+2] (exclusive prefix sums, offsets[E+1] = the pairs placed),
 * perm [T*k + T*has_shared] (pair ids in bucket order, then -1 past offsets[E+1]).
 * Every topk_ids value must lie in [0, E) or be -1 (an omitted pair: in no bucket). */
int moe_bucket(const moe_layer *L, const int32_t *topk_ids, int32_t T, int32_t *counts,
               int32_t *offsets, int32_t *perm, void *ws, size_t ws_bytes, void *stream);

/* The whole layer: y [T][H] fp32.  The dbg_* outputs are optional (NULL: not
 * written): the routing and bucketing the call used, in the shapes above.
 * path is a moe_path. */
int moe_forward(const moe_layer *L, const void *x, int32_t x_dtype, int32_t T, float *y,
                void *ws, size_t ws_bytes, void *stream, int32_t path, int32_t *dbg_ids,
                float *dbg_w, int32_t *dbg_counts, int32_t *dbg_offsets, int32_t *dbg_perm);

/* Bytes of the scratch array moe_forward_noalloc uses on each device (32 MiB). */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/* moe_forward for callers that cannot allocate or pass a workspace (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same kernels and
 * the same y bits, with the workspace taken from a scratch array of
 * MOE_NOALLOC_SCRATCH_BYTES that the library holds on each device it runs on (from the
 * device's first call until the process ends).  Calls nothing that allocates.
 * Arguments and errors as for moe_forward (no debug outputs), plus MOE_ERR_WORKSPACE
 * when moe_workspace_bytes(L, T) exceeds MOE_NOALLOC_SCRATCH_BYTES (decode batches of
 * every shape here fit; prefill chunks of a few hundred tokens do) and MOE_ERR_HIP when
 * the scratch's address cannot be obtained.  The first call on a device also enqueues a
 * clear of the scratch's synchronisation header on `stream`.
 * All calls on one device share the one array: calls that overlap in time on the same
 * device (different streams, threads or processes sharing the device's code object)
 * race and give undefined results; serialise them (one stream, or events). */
int moe_forward_noalloc(const moe_layer *L, const void *x, int32_t x_dtype, int32_t T, float *y, void *stream,
                        int32_t path);

/* Stages of one forward call, for moe_forward_timed. */
typedef enum {
  MOE_STAGE_ROUTER = 0,   /* router logits */
  MOE_STAGE_TOPK = 1,     /* top-k and gates */
  MOE_STAGE_BUCKET = 2,   /* bucketing by expert */
  MOE_STAGE_GATEUP = 3,   /* fused dequant + gate/up + SwiGLU */
  MOE_STAGE_DOWN = 4,     /* dequant + down projection */
  MOE_STAGE_COMBINE = 5,  /* gate-weighted combine */
  MOE_STAGE_ACT_QUANT = 6,  /* fp8 activation planes (MXFP4 prefill path) */
  MOE_NUM_STAGES = 7
} moe_stage;

/* moe_forward with per-stage timing: stage_events holds 2*MOE_NUM_STAGES hipEvent_t
 * handles (created by the caller with timing enabled; any may be NULL).  Event
 * 2s / 2s+1 is stamped at the start / end of the kernel that runs stage s, by the
 * dispatch packet itself, so hipEventElapsedTime gives that kernel's execution
 * time.  A stage fused into another kernel on the chosen path leaves its events
 * untouched.  No debug outputs. */
int moe_forward_timed(const moe_layer *L, const void *x, int32_t x_dtype, int32_t T, float *y,
                      void *ws, size_t ws_bytes, void *stream, int32_t path,
                      void *const *stage_events);

/* Test export: decode one packed matrix (layout above) to fp32 out [rows][cols],
 * bit-exact (every element is exactly representable in fp32 for MXFP4 scales
 * u <= 252 and every finite fp16 scale; AFF3 gives the fp32 rounding of the exact
 * scale * q + bias).  codebook: CB4 [16] int8, NULL otherwise.
 * Errors: MOE_ERR_INVALID_ARG for an unknown format, rows not a positive multiple of
 * 16, cols not a positive multiple of 32, NULL packed/out, or a CB4 call without a
 * codebook; MOE_ERR_UNSUPPORTED above 2^34 elements; MOE_ERR_ALIGNMENT for packed or
 * out not 16-byte aligned. */
int moe_dequant(int32_t wfmt, const void *packed, const int8_t *codebook, int32_t rows,
                int32_t cols, float *out, void *stream);

/* Test export of the grouped (prefill) path's CB4 decode: the same matrix decoded through
 * the grouped kernels' own replicated codebook table and lookup, to the same bit-exact
 * fp32 values as moe_dequant.  (The grouped MXFP4 kernels feed the stored E2M1 codes and
 * E8M0 scales to the block-scaled matrix instruction as they are, so they decode nothing.)
 * Errors: MOE_ERR_UNSUPPORTED for a format other than MOE_WFMT_CB4; otherwise as
 * moe_dequant. */
int moe_dequant_grouped(int32_t wfmt, const void *packed, const int8_t *codebook, int32_t rows,
                        int32_t cols, float *out, void *stream);

/* Helper between stacked layers (not part of the layer):
 * x_next[t][n] = bf16_rne(y[t][n] / sqrt(mean_n y[t][n]^2 + eps)), bf16 bits.
 * The sum of squares (exact squares, summed in a fixed order), the mean, the square
 * root and the quotient are fp64 (the square root and quotient correctly rounded), and
 * the fp64 quotient is rounded once to bf16 (nearest, ties to even).  y is [T][H] fp32;
 * eps >= 0 (converted exactly to fp64); results of magnitude below 2^-126 (the bf16
 * normal range) are outside this definition.  Errors: MOE_ERR_INVALID_ARG for T < 0,
 * H <= 0, eps < 0 or NaN, or a NULL pointer with T > 0. */
int moe_rms_rescale(const float *y, int32_t T, int32_t H, float eps, void *x_next_bf16,
                    void *stream);

/* The whole layer on the RMS rescale of the previous layer's output.
 * x = the bf16 values moe_rms_rescale(y_prev, T, H, eps) writes; then moe_forward of x as
 * MOE_BF16, with the same routing, kernels and y bits.
 * residual = 1: y = y_prev + that layer output (the pre-norm block's residual add,
 * added in fp32 after the fixed-order combine); residual = 0: y = the layer output.
 * Below 8 tokens on the decode kernels (and T*H <= 24576) the rescale is folded into the
 * router kernel, which also writes x for the projections, saving the separate launch.  The router
 * kernels of "How Neural runs a 120-billion-parameter model on one gaming PC" likewise
 * hand on the normalized hidden state with the expert ids and weights (section "How one
 * token and one prompt are processed", step 2).
 * Otherwise the rescale kernel runs first.
 * Arguments:
 *   y_prev        [T][H] fp32, 16-byte aligned, must not be y;
 *   eps           >= 0;
 *   residual      0 or 1;
 *   path          as for moe_forward;
 *   stage_events  as for moe_forward_timed, or NULL.
 * Workspace: moe_workspace_bytes(L, T).  Errors as for moe_forward;
 * MOE_ERR_INVALID_ARG also for eps < 0 or NaN, residual not 0 or 1, or y_prev == y. */
int moe_forward_rms(const moe_layer *L, const float *y_prev, float eps, int32_t residual, int32_t T,
                    float *y, void *ws, size_t ws_bytes, void *stream, int32_t path,
                    void *const *stage_events);

/* Measurement helper (not part of the layer): reads `bytes` (a multiple of 16) of buf
 * with 16-byte nontemporal loads, grid-stride over `blocks` blocks of 256 threads, and
 * writes one word per block to out[blocks] (the xor of what it read).  Timing it gives
 * the HBM read bandwidth a plain stream achieves on this GPU.  Errors:
 * MOE_ERR_INVALID_ARG for NULL pointers, bytes 0 or not a multiple of 16, blocks
 * outside 1 .. 2^20; MOE_ERR_ALIGNMENT for buf not 16-byte or out not 4-byte aligned. */
int moe_hbm_read_probe(const void *buf, size_t bytes, uint32_t *out, int32_t blocks, void *stream);

/* [host] Static description of a status code. */
const char *moe_status_str(int status);

#ifdef __cplusplus
}
#endif
#endif /* MOEQ_H */
