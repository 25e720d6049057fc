/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention forward library.
 *
 * One operation is exported: the chunked (16-token) forward pass of Kimi Delta
 * Attention with a 128 x 128 state per (sequence, head). It computes, for each
 * sequence and head, token by token (Doubleword page "You Could Have Come Up
 * with Kimi Delta Attention", section 4, boxed KDA equations):
 *
 *     S~ = S Diag(alpha_t);  e = beta_t (v_t - S~ k_t);  S = S~ + e k_t^T;
 *     o_t = S (scale * q_t)
 *
 * after the activations the FlashKDA pages describe (instagit FlashKDA summary,
 * "Chunked Token Processing"; DocSearch FlashKDA digest, "Configure
 * fla_chunk_kda"): alpha_t = exp(lower_bound * sigmoid(g_raw_t)) per key
 * channel, beta_t = sigmoid(beta_raw_t), and q_t, k_t L2-normalised per token
 * as x / sqrt(sum x^2 + 1e-6). It is evaluated with the chunkwise method of the
 * same Doubleword page, section 6, either split into a chunk-parallel kernel
 * and a per-(sequence, head) recurrence kernel, or in one single-pass kernel
 * per (sequence, head) (see KDA_FLAG_SPLIT / KDA_FLAG_FUSED); short sequences
 * and decode steps run the section 4 recurrence token by token
 * (KDA_FLAG_RECURRENT).
 *
 * Conventions for every entry point:
 *  - Pointers named "device" point to GPU memory; all others to host memory.
 *  - The caller owns every buffer. The library never allocates, frees or
 *    synchronises, and keeps no global mutable state: calls are reentrant and
 *    thread-safe as long as they do not share output or workspace buffers.
 *  - Work is enqueued on the caller's HIP stream (passed as void*, NULL = the
 *    null stream) and the call returns after enqueueing.
 *  - All arguments are checked before anything is enqueued; a call that
 *    returns an error has launched nothing and written nothing.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Head dimension K = V (the only one supported; DocSearch FlashKDA digest,
 * "flash_kda.fwd API reference": K = V = 128). */
#define KDA_HEAD_DIM 128
/* Tokens per chunk (FlashKDA v1 deep-dive, section 1, "Chunk Size Selection"). */
#define KDA_CHUNK 16
/* Required alignment of the workspace base, in bytes (instagit FlashKDA
 * summary, "State Management and Workspace Allocation": 128-byte aligned
 * intermediate buffers). */
#define KDA_WORKSPACE_ALIGN 128
/* Accepted lower_bound range (the gate is g = lower_bound * sigmoid(g_raw);
 * the pages use -5, FlashKDA review section 2.1). */
#define KDA_LOWER_BOUND_MIN (-10.0f)
#define KDA_LOWER_BOUND_MAX (0.0f)
/* Largest lower_bound accepted with KDA_FLAG_BF16_RESIDENT_STATE. */
#define KDA_BF16_RESIDENT_MAX_LOWER_BOUND (-0.2f)

typedef enum kda_status {
    KDA_OK = 0,
    KDA_ERR_NULL_ARG = 1,    /* a required pointer is NULL                          */
    KDA_ERR_BAD_SHAPE = 2,   /* head_dim != 128, H outside [1, 65535], B/T/N out of
                                range, or a launch of the chosen path would exceed
                                the device's grid limits (2^32 work-items along x;
                                e.g. the token-by-token path from 2^22 (sequence,
                                head) pairs, the single pass from about 6.1 M)     */
    KDA_ERR_BAD_DTYPE = 3,   /* unknown dtype code                                  */
    KDA_ERR_BAD_SEQLENS = 4, /* cu_seqlens given with batch != 1, or N < 1           */
    KDA_ERR_BAD_ARG = 5,     /* lower_bound / scale out of range or non-finite,
                                unknown or conflicting flag bits, or out aliasing
                                an input                                           */
    KDA_ERR_WORKSPACE = 6,   /* workspace NULL, too small, or not 128-B aligned     */
    KDA_ERR_MISALIGNED = 7,  /* a tensor base address is not 16-B aligned           */
    KDA_ERR_HIP = 8,         /* a kernel launch failed (HIP runtime error)          */
    KDA_ERR_TOO_LARGE = 9    /* kda_fwd_noalloc: the call needs more scratch than
                                the library's static buffer holds (more than
                                KDA_NOALLOC_MAX_SEQS sequences)                    */
} kda_status_t;

/* Element types. */
typedef enum kda_dtype {
    KDA_DTYPE_BF16 = 0,
    KDA_DTYPE_FP32 = 1
} kda_dtype_t;

/* Flag bits for kda_desc_t.flags. */
enum {
    /* Use the fp32 reference kernels (no bf16 matrix-core operands) even for
     * bf16 I/O. fp32 I/O always uses them. */
    KDA_FLAG_FP32_COMPUTE = 1u,
    /* bf16-compute kda_fwd: run the two-kernel path (chunk-parallel kernel
     * writing the workspace, then the recurrence kernel), which is what
     * kda_fwd_prepare + kda_fwd_recur run. With fewer than 96 (sequence, head)
     * pairs (and without KDA_FLAG_BF16_RESIDENT_STATE) the recurrence runs in
     * look-ahead form and the workspace also holds 4096 B per (chunk, head);
     * kda_fwd_workspace_size accounts for it. */
    KDA_FLAG_SPLIT = 2u,
    /* bf16-compute kda_fwd: run the single-pass kernel (one workgroup per
     * (sequence, head) prepares each chunk in on-chip memory and runs the
     * recurrence on it; the workspace holds only the chunk map and the order
     * in which the workgroups take the sequences, longest first). Not valid
     * with fp32 compute, with KDA_FLAG_SPLIT, or for kda_fwd_prepare /
     * kda_fwd_recur. */
    KDA_FLAG_FUSED = 4u,
    /* kda_fwd: run the token-by-token kernel (the boxed recurrence in fp32,
     * one token after another, for decode and short sequences; any io and
     * state dtype; the workspace holds only the chunk map). Not valid with
     * KDA_FLAG_SPLIT or KDA_FLAG_FUSED, or for kda_fwd_prepare /
     * kda_fwd_recur. */
    KDA_FLAG_RECURRENT = 8u,
    /* g_raw holds one gate per token and head, [B*T][H] like beta_raw (only
     * element-aligned), applied to every key channel: alpha_t is then
     * exp(lower_bound * sigmoid(g_raw_t)) times the all-ones vector, the
     * Gated DeltaNet special case of the recurrence (Doubleword page, section
     * 3). Valid with every path. */
    KDA_FLAG_SCALAR_GATE = 16u,
    /* Two-kernel bf16 path with a bf16-resident recurrent state: the
     * recurrence rounds its state to bf16 when loading it and after every
     * chunk's fp32 update, as a kernel that keeps the on-chip state in bf16
     * between updates does (FlashKDA deep-dive, section 3), instead of
     * carrying it in fp32. For measuring that choice; implies the two-kernel
     * path and is not valid with fp32 compute or another path flag. Its
     * roundings accumulate when the state barely decays: with lower_bound
     * above KDA_BF16_RESIDENT_MAX_LOWER_BOUND the call is rejected with
     * KDA_ERR_BAD_ARG (at lower_bound 0 the final state measured 1.04 times
     * the bf16 tolerance, at -0.2 0.36 times). */
    KDA_FLAG_BF16_RESIDENT_STATE = 32u,
    /* bf16-compute kda_fwd: run the segmented single pass, for few (sequence,
     * head) pairs over long sequences. Every sequence is cut into
     * max(2, 256 / (num_seqs * num_heads)) segments (from the average
     * sequence; at least 8 chunks each, the first half again as long as the
     * others), so that about 256 (segment, head) workgroups, one per compute
     * unit, run at once. Each segment runs the single-pass kernel twice over the
     * same prepared chunks: from a zero state (the first segment: the initial
     * state) with the inputs, and from the identity with v = 0, which gives
     * the segment's key-space transfer (the product form of the transition,
     * Doubleword page, section 4.1). A scan over the segments then forms each
     * segment's true incoming state and the final state, and a last kernel
     * adds the incoming state's contribution to the outputs. The workspace
     * holds the chunk map, three 64 KiB [128][128] matrices per (segment, head)
     * (the segment's final state from zero, its transfer as split bf16, the
     * true incoming state) and 4 KiB of bf16 per (chunk, head) for the
     * transfer applied to the queries. Not valid with fp32 compute, another
     * path flag or KDA_FLAG_BF16_RESIDENT_STATE, or for kda_fwd_prepare /
     * kda_fwd_recur. */
    KDA_FLAG_SEGMENTED = 64u
};
/* Without a path flag, kda_fwd runs the token-by-token kernel when the
 * sequences average at most KDA_RECURRENT_MAX_AVG_TOKENS tokens (batch mode:
 * seqlen; packed: T_tot / num_seqs), else, for bf16 compute, the segmented
 * single pass when num_seqs * num_heads <= KDA_SEGMENTED_MAX_PAIRS and the
 * sequences average at least KDA_SEGMENTED_MIN_AVG_CHUNKS 16-token chunks
 * (chunk bound / num_seqs; KDA_SEGMENTED_MIN_AVG_CHUNKS_FEW_PAIRS up to
 * KDA_SEGMENTED_FEW_PAIRS pairs), else the
 * single-pass kernel when
 * num_seqs * num_heads >= KDA_FUSED_MIN_PAIRS or the sequences average at
 * most KDA_FUSED_MAX_AVG_CHUNKS chunks, and the two-kernel path otherwise;
 * fp32 compute uses
 * the fp32 two-kernel path. The thresholds are where each path measured
 * fastest on MI355X. The paths evaluate the same chunkwise equations and
 * agree to bf16 rounding; they are not bitwise identical (the single pass
 * applies the L2 normalisation after its in-chunk products instead of
 * before). */
#define KDA_FUSED_MIN_PAIRS 64
#define KDA_FUSED_MAX_AVG_CHUNKS 8
#define KDA_SEGMENTED_MAX_PAIRS 128
#define KDA_SEGMENTED_MIN_AVG_CHUNKS 56
#define KDA_SEGMENTED_FEW_PAIRS 80
#define KDA_SEGMENTED_MIN_AVG_CHUNKS_FEW_PAIRS 40
#define KDA_RECURRENT_MAX_AVG_TOKENS 4

/*
 * Problem description (host memory).
 *
 * Layouts (all row-major, DocSearch FlashKDA digest "flash_kda.fwd API
 * reference"; instagit FlashKDA summary "Chunked Token Processing"):
 *   q, k, g_raw, v, out : [B*T][H][128]  (batch rows flattened; with
 *                          cu_seqlens B = 1 and the T_tot tokens are packed)
 *   beta_raw            : [B*T][H]  (g_raw too with KDA_FLAG_SCALAR_GATE)
 *   initial/final state : [N][H][128 (value channel V)][128 (key channel K)]
 *
 * Without cu_seqlens every batch row is an independent sequence of length
 * seqlen and num_seqs must equal batch. With cu_seqlens, batch must be 1,
 * seqlen is T_tot and cu_seqlens holds num_seqs + 1 int32 token offsets.
 */
typedef struct kda_desc {
    int64_t batch;       /* B >= 1                                           */
    int64_t seqlen;      /* T >= 0 per batch row, or T_tot with cu_seqlens    */
    int64_t num_seqs;    /* N >= 1 (== batch without cu_seqlens)              */
    int32_t num_heads;   /* H in [1, 65535]                                   */
    int32_t head_dim;    /* must be KDA_HEAD_DIM                              */
    int32_t io_dtype;    /* kda_dtype_t of q, k, v, g_raw, beta_raw and out   */
    int32_t state_dtype; /* kda_dtype_t of initial_state and final_state      */
    float scale;         /* read scale s, finite and > 0 (usually 128^-1/2)   */
    uint32_t flags;      /* KDA_FLAG_* bits                                   */
} kda_desc_t;

/*
 * Bytes of device workspace kda_fwd needs for this description (a pure host
 * function; no GPU call). The size is an upper bound computed from B, T, N
 * and H only, because the chunk count of a packed batch depends on device-side
 * cu_seqlens: at most (T_tot + 15 N) / 16 chunks. Unless flags hold
 * KDA_FLAG_FUSED, KDA_FLAG_RECURRENT or KDA_FLAG_SEGMENTED, it covers the
 * two-kernel path, so the same workspace also serves kda_fwd_prepare /
 * kda_fwd_recur, and also the segmented single pass when kda_fwd would pick
 * it; with KDA_FLAG_RECURRENT it is only the chunk map (a few hundred bytes
 * plus 8 (N + 1)), with KDA_FLAG_FUSED the chunk map and the order in which the
 * single pass takes the sequences (longest first, 4 N more), with
 * KDA_FLAG_SEGMENTED the segmented pass's workspace. Returns 0 if the
 * description itself is invalid (NULL, bad shape, dtype or flags).
 */
size_t kda_fwd_workspace_size(const kda_desc_t *desc);

/*
 * Forward pass.
 *   q, k, v, g_raw : device, io_dtype, [B*T][H][128] (g_raw: [B*T][H] with
 *                    KDA_FLAG_SCALAR_GATE)
 *   beta_raw       : device, io_dtype, [B*T][H]
 *   cu_seqlens     : device int32 [N+1] token offsets, or NULL (batch mode).
 *                    Contents are the caller's contract (cu_seqlens[0] = 0,
 *                    non-decreasing, cu_seqlens[N] = T_tot). The kernels clamp
 *                    them into that form before use, so bad contents can give
 *                    wrong results but never out-of-bounds accesses; the first
 *                    int32 of the workspace is set to 1 if the offsets were
 *                    valid and 0 if they had to be clamped.
 *   initial_state  : device, state_dtype, [N][H][128][128], or NULL (= zeros)
 *   out            : device, io_dtype, like v; must not overlap any input
 *   final_state    : device, state_dtype, [N][H][128][128], or NULL (not
 *                    written). May be the same buffer as initial_state
 *                    (in-place streaming); partial overlap is not allowed.
 *   lower_bound    : gate bound in [KDA_LOWER_BOUND_MIN, KDA_LOWER_BOUND_MAX]
 *   desc           : host, problem description
 *   workspace      : device, >= kda_fwd_workspace_size(desc) bytes, 128-B
 *                    aligned; contents on entry are ignored
 *   stream         : hipStream_t, or NULL for the null stream
 * Tensor bases must be 16-B aligned (beta_raw, and a scalar g_raw: element-aligned).
 * A sequence of length 0 gets final_state = initial_state (or zeros).
 * B*T = 0 with batch mode is a no-op apart from writing final_state.
 */
kda_status_t kda_fwd(const void *q, const void *k, const void *v,
                     const void *g_raw, const void *beta_raw,
                     const int32_t *cu_seqlens,
                     const void *initial_state,
                     void *out, void *final_state,
                     float lower_bound,
                     const kda_desc_t *desc,
                     void *workspace, size_t workspace_bytes,
                     void *stream);

/*
 * The two stages of kda_fwd, for callers that time or overlap them: the
 * chunk-parallel stage (chunk map, gate, in-chunk log-decay prefix sums, L2
 * norms, the decayed 16 x 16 blocks, the unit-lower-triangular inverse and
 * the decayed key/query operands; Doubleword KDA page, sections 6.1-6.3 and
 * 6.6) writes the workspace; the recurrence stage (the chunk-state scan with
 * outputs, sections 6.4-6.5) reads it and writes out and final_state.
 * kda_fwd(args) on the two-kernel path (see KDA_FLAG_SPLIT) is exactly
 * kda_fwd_prepare(args) followed by kda_fwd_recur(args). Both take kda_fwd's
 * arguments with the same meaning and checks (KDA_FLAG_FUSED and
 * KDA_FLAG_RECURRENT are rejected with KDA_ERR_BAD_ARG); recur must see the workspace written by a prepare call
 * with the same arguments, ordered before it (same stream, or an event). Each
 * returns after enqueueing its kernels.
 */
kda_status_t kda_fwd_prepare(const void *q, const void *k, const void *v,
                             const void *g_raw, const void *beta_raw,
                             const int32_t *cu_seqlens,
                             const void *initial_state,
                             void *out, void *final_state,
                             float lower_bound,
                             const kda_desc_t *desc,
                             void *workspace, size_t workspace_bytes,
                             void *stream);
kda_status_t kda_fwd_recur(const void *q, const void *k, const void *v,
                           const void *g_raw, const void *beta_raw,
                           const int32_t *cu_seqlens,
                           const void *initial_state,
                           void *out, void *final_state,
                           float lower_bound,
                           const kda_desc_t *desc,
                           void *workspace, size_t workspace_bytes,
                           void *stream);

/*
 * The two stages of kda_fwd on the segmented single pass (see
 * KDA_FLAG_SEGMENTED), for callers that time them: kda_fwd_seg_pass runs the
 * chunk map and the single-pass kernel over every (segment, head), writing
 * out (complete for each sequence's first segment, without the incoming
 * state's share elsewhere) and the segments' states, transfers and y vectors
 * into the workspace; kda_fwd_seg_finish scans the segments (true incoming
 * states, final_state) and adds each incoming state's share to out. On that
 * path kda_fwd(args) is exactly kda_fwd_seg_pass(args) followed by
 * kda_fwd_seg_finish(args), ordered as kda_fwd_prepare / kda_fwd_recur are.
 * Both take kda_fwd's arguments with the same meaning and checks, run the
 * segmented stages whether or not desc->flags holds KDA_FLAG_SEGMENTED, and
 * reject any other path flag, KDA_FLAG_BF16_RESIDENT_STATE and fp32 compute
 * with KDA_ERR_BAD_ARG. The workspace must be the size kda_fwd_workspace_size
 * reports with KDA_FLAG_SEGMENTED.
 */
kda_status_t kda_fwd_seg_pass(const void *q, const void *k, const void *v,
                              const void *g_raw, const void *beta_raw,
                              const int32_t *cu_seqlens,
                              const void *initial_state,
                              void *out, void *final_state,
                              float lower_bound,
                              const kda_desc_t *desc,
                              void *workspace, size_t workspace_bytes,
                              void *stream);
kda_status_t kda_fwd_seg_finish(const void *q, const void *k, const void *v,
                                const void *g_raw, const void *beta_raw,
                                const int32_t *cu_seqlens,
                                const void *initial_state,
                                void *out, void *final_state,
                                float lower_bound,
                                const kda_desc_t *desc,
                                void *workspace, size_t workspace_bytes,
                                void *stream);

/*
 * kda_fwd without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation). It takes kda_fwd's other arguments with the same meaning
 * and checks, and runs only the paths whose scratch is small: the single-pass
 * kernel (KDA_FLAG_FUSED, and without a path flag for bf16 compute) or the
 * token-by-token kernel (KDA_FLAG_RECURRENT, and without a path flag for
 * sequences averaging at most KDA_RECURRENT_MAX_AVG_TOKENS tokens or for fp32
 * compute). Their scratch -- the chunk map and the order of the sequences --
 * lives in a static device buffer of KDA_NOALLOC_SCRATCH_BYTES that the library
 * holds on each GPU it runs on until the process ends; its address is looked
 * up once per device, on the first call with that device current. The call
 * allocates and frees nothing.
 *  - KDA_FLAG_SPLIT, KDA_FLAG_SEGMENTED and KDA_FLAG_BF16_RESIDENT_STATE give
 *    KDA_ERR_BAD_ARG; more than KDA_NOALLOC_MAX_SEQS sequences give
 *    KDA_ERR_TOO_LARGE; both before anything is enqueued.
 *  - Every call on one GPU uses that GPU's one buffer: calls that overlap in
 *    time on one GPU (different streams, or host threads) race and must be
 *    serialised by the caller. Nothing in the buffer needs clearing between
 *    calls: each call rewrites what it reads.
 */
#define KDA_NOALLOC_MAX_SEQS 65536
#define KDA_NOALLOC_SCRATCH_BYTES (800u * 1024u)
kda_status_t kda_fwd_noalloc(const void *q, const void *k, const void *v,
                             const void *g_raw, const void *beta_raw,
                             const int32_t *cu_seqlens,
                             const void *initial_state,
                             void *out, void *final_state,
                             float lower_bound,
                             const kda_desc_t *desc,
                             void *stream);

/* Static, human-readable name of a status code (never NULL). */
const char *kda_status_str(kda_status_t status);

/* Library version as major * 10000 + minor * 100 + patch. */
int kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
