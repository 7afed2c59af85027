/*
 * kdkl.h -- C ABI of libkdkl: the fused chunked top-K KL distillation loss over the LM head,
 * forward and backward, on one AMD Instinct MI355X (gfx950).
 *
 * What it computes. The teacher side is an offline cache: for each sequence position, the
 * K most probable teacher tokens and their logits, computed once and reused. Sources:
 * "Making knowledge distillation cheap enough to run in production" (aiexpert.news),
 * paragraph on the first fix (offline distillation); dailyai.com.br launch note, section
 * "As duas inovacoes", item 1.
 *
 * The student side is the LM head applied to the student's last hidden states. The loss is
 * the Kullback-Leibler divergence from the teacher's top-K distribution to the student's
 * full-vocabulary distribution. Its fused chunked form projects one piece of the hidden
 * states at a time, folds it into a running accumulator, discards it, and recomputes it in
 * the backward pass. Source: same aiexpert.news article, paragraph on the second fix and
 * its three equivalent formulations.
 *
 * It is a drop-in KL term: inputs are hidden states and the head weight, and nothing about
 * the model changes. Source: same article, paragraph on the integration surface.
 *
 * With
 *   H [N,d]    student hidden states, row-major (N = batch * sequence rows);
 *   W [V,d]    LM-head weight, row-major (the layout of a torch nn.Linear(d, V) weight);
 *   idx [N,K]  cached teacher token ids (int32, distinct within a row, in [0,V));
 *   t [N,K]    cached teacher logits;
 *   T          temperature;
 *   z = H W^T  student logits, never stored whole;
 *   u = z/T    tempered student logits;
 *   lse_n = log sum_v exp(u_nv);
 *   p_t = softmax(t/T) over the K cached entries (the tail beyond the top-K is dropped);
 *   KL_n = sum_k p_t[n,k] * (log p_t[n,k] - u[n,idx[n,k]] + lse_n);
 *   loss = T^2 / n_norm * sum_n KL_n;
 *   with g = d(outer loss)/d(loss), the backward is
 *     G = g * T / n_norm * (softmax(u) - P_t), P_t = p_t scattered at idx, zero elsewhere;
 *     dH = G W;
 *     dW = G^T H.
 *
 * Readings of points the pages leave open:
 *   - KL direction is teacher -> student;
 *   - temperature enters both sides and the loss carries T^2;
 *   - the mean is over n_norm rows;
 *   - the student is normalised over all V tokens.
 *
 * Conventions shared by every call:
 *   - Memory: every pointer argument except `p` is device memory on the current HIP
 *     device, allocated and owned by the caller. `p` is host memory. The library never
 *     allocates or frees device memory, and no result depends on an earlier call. Host-side
 *     state is limited to the optional timing (kd_timing_*: a process-wide pool of HIP events
 *     and running totals under a mutex) and a per-device cache of the compute-unit count.
 *     Calls that do not share output or workspace buffers may run concurrently on different
 *     streams.
 *   - Streams: work is enqueued on `stream`, an hipStream_t (NULL means the null stream).
 *     Outputs are valid once the caller has synchronised that stream. No call synchronises,
 *     except as noted for KD_VALIDATE_IDX.
 *   - Errors: arguments are checked on the host before anything is enqueued, and a bad
 *     argument returns its kd_status at once with nothing written. A launch failure returns
 *     KD_ERR_HIP. A fault inside a kernel surfaces at the caller's next synchronisation of
 *     the stream. No C++ exception crosses this interface.
 *   - Preconditions the host cannot check without reading device memory: idx in [0,V) and
 *     distinct within each row. An out-of-range id is never dereferenced (no fault), but the
 *     zk slot of that entry is left unwritten, so the KL_n and zk of its row, and the loss,
 *     are undefined; repeated ids give undefined values for their row. Set KD_VALIDATE_IDX
 *     (or run kd_validate_ids) to have the ids checked.
 *   - Teacher logits: finite, or -inf for a masked entry. A -inf entry has p_t = 0: it adds
 *     nothing to KL_n (0 log 0 = 0) and nothing is subtracted at its id in the gradient. Every
 *     row needs at least one finite cached logit; +inf or NaN logits give undefined values.
 *   - Alignment: H, W, dH and dW must be 16-byte aligned (KD_ERR_VALUE otherwise).
 *   - Workspace: the caller passes ws (256-byte aligned) of at least the bytes returned by
 *     the matching *_workspace_bytes query for the same problem. Its contents on entry do not
 *     matter; on return they are unspecified.
 */
#ifndef KDKL_H
#define KDKL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 1: first release. 2: kd_validate_ids added; chunks capped at 2^20 rows; kd_dense_kl limited
 * to V <= 2^21. 3: KD_LOW_MEMORY and kd_chunked_logits added; a -inf teacher logit counts as a
 * masked entry. 4: kd_fused_kl_fwd_noalloc added. Calls and structures of earlier versions are
 * unchanged. */
#define KDKL_ABI_VERSION 4

/* Same type as hipStream_t; declared here so that this header does not need the HIP headers. */
typedef struct ihipStream_t* kd_stream;

typedef enum kd_status {
    KD_OK = 0,
    KD_ERR_NULL = 1,      /* a required pointer is NULL */
    KD_ERR_SHAPE = 2,     /* N, d, V, K or chunk out of the supported range */
    KD_ERR_DTYPE = 3,     /* unknown or unsupported dtype */
    KD_ERR_VALUE = 4,     /* T not finite and > 0, n_norm not finite, unknown flag, or a
                             H, W, dH or dW pointer not 16-byte aligned */
    KD_ERR_WORKSPACE = 5, /* ws_bytes smaller than the query, or ws not 256-byte aligned */
    KD_ERR_INDEX = 6,     /* KD_VALIDATE_IDX found an id out of range or repeated in a row */
    KD_ERR_HIP = 7,       /* the HIP runtime reported an error while enqueueing */
    KD_ERR_INTERNAL = 8
} kd_status;

typedef enum kd_dtype {
    KD_FP32 = 0,
    KD_BF16 = 1
} kd_dtype;

/* flags */
#define KD_VALIDATE_IDX  0x1u /* check idx on the device first; this syncs the stream once
                                 (kd_validate_ids is the same check without the sync) */
#define KD_ACCUMULATE_DW 0x2u /* kd_fused_kl_bwd / kd_dense_kl add into dW instead of overwriting */
#define KD_SKIP_DW       0x4u /* kd_fused_kl_bwd computes dH only (dW may be NULL): for a frozen head.
                                 Ignored by kd_fused_kl_fwd; KD_ERR_VALUE for the other calls and
                                 together with KD_ACCUMULATE_DW */
#define KD_LOW_MEMORY    0x8u /* memory-lean fused calls: of the default backward's buffers the
                                 workspace keeps the chunk's gradient tile G_c [chunk, V], and none
                                 of the transposed or stage-tiled copies of W, G_c and H_c (nor the
                                 forward's stage-tiled copies of W and H); dH and dW then read
                                 their operands as stored, on a slower GEMM path, with one dW pass
                                 per chunk. Same results up to rounding order. Changes
                                 kd_fused_workspace_bytes; KD_ERR_VALUE for the other loss calls */

/*
 * Problem descriptor (host memory).
 *   N, d, V, K   sizes as above; limits: N >= 1, 8 <= d <= 1048576 and d % 8 == 0, 1 <= V <= 4194304,
 *                1 <= K <= min(V, 1024), N * K < 2^31, N * d < 2^31, V * d < 2^31. The backward
 *                calls (kd_fused_kl_bwd without KD_LOW_MEMORY, kd_chunked_kl, kd_fused_kl_fwdbwd)
 *                also need V <= 3355392 (bf16) or V <= 1677568 (fp32), and kd_fused_kl_bwd with
 *                KD_LOW_MEMORY in bf16 V <= 4194048: KD_ERR_SHAPE otherwise.
 *   chunk        rows per backward chunk (>= 1; N need not be a multiple). It bounds the
 *                backward's per-chunk gradient tile G_c [chunk, V] in the workspace. The
 *                forward keeps each projected tile in registers only, so its memory does not
 *                depend on chunk. Values above 1048576 (2^20) are taken as 2^20, which keeps
 *                the chunk-strided operands of the dW product within 32-bit buffer offsets;
 *                the chunk changes memory use and summation order only, never the result.
 *   T            temperature, finite and > 0.
 *   n_norm       denominator of the mean; <= 0 means N. Set it to the global row count when
 *                one batch is split over several calls.
 *   act          dtype of H, W and dH: KD_BF16 (fp32 accumulation) or KD_FP32 (fp32 products).
 *   tlogit       dtype of the cached teacher logits t: KD_BF16 or KD_FP32.
 *   flags        KD_VALIDATE_IDX | KD_ACCUMULATE_DW | KD_SKIP_DW | KD_LOW_MEMORY.
 */
typedef struct kd_problem {
    int64_t N;
    int64_t d;
    int64_t V;
    int64_t K;
    int64_t chunk;
    float T;
    float n_norm;
    int32_t act;
    int32_t tlogit;
    uint32_t flags;
    uint32_t reserved; /* must be 0 */
} kd_problem;

/* ABI version of the loaded library (KDKL_ABI_VERSION it was built with). */
int kd_abi_version(void);

/* Static English text for a status code; never NULL. */
const char* kd_status_str(kd_status s);

/* Workspace bytes for kd_fused_kl_fwd and kd_fused_kl_bwd (one query serves both). Grows
 * with N only through O(N*K) and O(N) terms; the rest is O(chunk * V + V * d). From N = 8192
 * rows (without KD_LOW_MEMORY) it includes copies of W and of a chunk of rows of H in a
 * stage-tiled layout, which the kernels read faster than W and H as stored (V * d elements of
 * the act dtype for W: 1.16 GB at V = 201,088, d = 2880 in bf16). Returns 0 if p is NULL or
 * invalid. */
size_t kd_fused_workspace_bytes(const kd_problem* p);

/*
 * Fused forward.
 *   H [N,d] act, W [V,d] act, idx [N,K] int32, tlog [N,K] tlogit       (inputs)
 *   loss [1] fp32      T^2/n_norm * sum_n KL_n                          (output)
 *   lse [N] fp32       logsumexp_v z_nv/T; the backward needs it        (output)
 *   row_kl [N] fp32    KL_n, or NULL to skip                            (output)
 *   zk [N,K] fp32      z at the cached ids, z[n, idx[n,k]], or NULL     (output)
 * Source: aiexpert.news "Making knowledge distillation cheap enough...", paragraph on the
 * three formulations (the fused chunked forward).
 */
kd_status kd_fused_kl_fwd(const kd_problem* p, const void* H, const void* W, const int32_t* idx,
                          const void* tlog, float* loss, float* lse, float* row_kl, float* zk,
                          void* ws, size_t ws_bytes, kd_stream stream);

/*
 * The fused forward for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation. Same arguments, checks and
 * results as kd_fused_kl_fwd (the same arithmetic, bit for bit; kd_fused_kl_fwd reads W and H
 * through stage-tiled copies in its workspace, this call as stored), without ws and ws_bytes: the
 * forward's workspace is a static device array of KD_NOALLOC_SCRATCH_BYTES inside the library,
 * one per GPU, held from the library's first use on that GPU until the process ends. The call
 * allocates nothing; the caller passes every input and output.
 *   Limit: the forward's share of kd_fused_workspace_bytes(p) without the tiled copies (O(N*K + N)
 *   bytes: at K = 100 and V = 201,088 about 815 bytes a row plus 1 MB, so N up to about 80,000
 *   rows) must fit in KD_NOALLOC_SCRATCH_BYTES, else
 *   KD_ERR_WORKSPACE with nothing enqueued. KD_VALIDATE_IDX gives KD_ERR_VALUE (it copies to the
 *   host and waits; run kd_validate_ids first instead).
 *   Calls on one GPU share its array: calls that overlap in time on one GPU (different streams
 *   or threads, unsynchronised) race and give undefined results. Nothing in the array needs to
 *   start at zero, so the contents an earlier call leaves do not matter.
 *   KD_ERR_HIP if the array's device address cannot be obtained.
 */
#define KD_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
kd_status kd_fused_kl_fwd_noalloc(const kd_problem* p, const void* H, const void* W, const int32_t* idx,
                                  const void* tlog, float* loss, float* lse, float* row_kl, float* zk,
                                  kd_stream stream);

/*
 * Fused backward: recomputes each chunk's logits instead of storing them.
 *   H, W, idx, tlog        as in the forward
 *   lse [N] fp32           from kd_fused_kl_fwd on the same inputs
 *   grad_loss [1] fp32     upstream gradient g of the scalar loss (device), or NULL for 1
 *   dH [N,d] act           written (overwritten)
 *   dW [V,d] fp32          overwritten, incremented under KD_ACCUMULATE_DW,
 *                          or untouched (and may be NULL) under KD_SKIP_DW
 * Source: same paragraph (the backward recomputes each chunk on the fly); dailyai.com.br
 * launch note, section "As duas inovacoes", item 2.
 */
kd_status kd_fused_kl_bwd(const kd_problem* p, const void* H, const void* W, const int32_t* idx,
                          const void* tlog, const float* lse, const float* grad_loss, void* dH,
                          float* dW, void* ws, size_t ws_bytes, kd_stream stream);

/* Workspace bytes for kd_dense_kl: two fp32 [N, V] grids (rounded up to whole tiles) plus a
 * small remainder. Returns 0 if p is NULL or invalid, or V exceeds the dense limit below. */
size_t kd_dense_workspace_bytes(const kd_problem* p);

/*
 * Dense formulation, forward and backward in one call, for memory and speed comparison.
 * It expands the cached teacher into a full [N, V] probability grid and compares it with the
 * full [N, V] student log-probability grid, so two vocabulary-by-sequence grids are resident
 * at once. Source: aiexpert.news article, paragraph on the three formulations (dense KL).
 *   Arguments as in the two fused calls; row_kl may be NULL. Same results up to rounding.
 *   Limit: V <= 2097152 (2^21), so that a tile's 256 rows of the logit grid stay within
 *   32-bit buffer offsets; KD_ERR_SHAPE above it (the fused calls take V up to 4194304).
 */
kd_status kd_dense_kl(const kd_problem* p, const void* H, const void* W, const int32_t* idx,
                      const void* tlog, const float* grad_loss, float* loss, float* lse,
                      float* row_kl, void* dH, float* dW, void* ws, size_t ws_bytes,
                      kd_stream stream);

/*
 * Forward-chunked formulation, forward and backward in one call. The teacher stays sparse and
 * the loss is computed one slice of rows at a time, but every student logit is kept (as z^T,
 * fp32, in the workspace) for the backward, which reads them instead of recomputing. Memory
 * therefore grows with N (4 * N * V bytes of logits) while the work drops to 6*N*d*V FLOPs.
 * Source: aiexpert.news "Making knowledge distillation cheap enough to run in production",
 * paragraph on the three formulations (forward-chunked KL: fastest, logits materialised for
 * the backward, memory still scaling with sequence length).
 *   Arguments as in kd_dense_kl; grad_loss (device scalar or NULL for 1) is applied to dH and
 *   dW; KD_ACCUMULATE_DW adds into dW. Same results as the fused calls up to rounding.
 */
size_t kd_chunked_workspace_bytes(const kd_problem* p);
kd_status kd_chunked_kl(const kd_problem* p, const void* H, const void* W, const int32_t* idx,
                        const void* tlog, const float* grad_loss, float* loss, float* lse,
                        float* row_kl, void* dH, float* dW, void* ws, size_t ws_bytes,
                        kd_stream stream);

/*
 * Where kd_chunked_kl keeps the student logits it materialises (the same paragraph: the
 * forward-chunked formulation stores the full logit grid for the backward). Host-only: it
 * enqueues nothing and reads no device memory. For a workspace `ws` of at least
 * kd_chunked_workspace_bytes(p) bytes, sets *zt to the fp32 array z^T [Vp][*ldzt] inside it
 * (Vp = V rounded up to a multiple of 256; element (v, n) = z[n, v] for n < N, v < V). After a
 * kd_chunked_kl call on the same p and ws has completed on its stream, the array holds that
 * call's logits, until the workspace is next written.
 *   Errors: as kd_chunked_kl's argument checks; KD_ERR_NULL if ws, zt or ldzt is NULL.
 */
kd_status kd_chunked_logits(const kd_problem* p, const void* ws, size_t ws_bytes, const float** zt,
                            int64_t* ldzt);

/*
 * Single-pass fused formulation: each chunk of rows is taken end to end (logits, its loss
 * terms, G_c, dH_c and its share of dW) and discarded before the next, so the logits are
 * computed once (6*N*d*V FLOPs instead of 8) and memory stays bounded by the chunk (the
 * chunk's fp32 logits, 4 * chunk * V bytes, on top of the fused backward's buffers). The
 * upstream gradient must be known at call time: grad_loss (device scalar or NULL for 1) is
 * applied to dH and dW. Source: aiexpert.news ticker "Multiverse Computing publishes efficient
 * KD technique cutting distillation VRAM", second change (sequence chunks processed end to
 * end and discarded after the backward pass).
 *   Arguments as in kd_dense_kl; KD_ACCUMULATE_DW adds into dW.
 */
size_t kd_fused_fwdbwd_workspace_bytes(const kd_problem* p);
kd_status kd_fused_kl_fwdbwd(const kd_problem* p, const void* H, const void* W, const int32_t* idx,
                             const void* tlog, const float* grad_loss, float* loss, float* lse,
                             float* row_kl, void* dH, float* dW, void* ws, size_t ws_bytes,
                             kd_stream stream);

/*
 * Offline top-K cache producer: the step before the loss, run once over the teacher's logits.
 * For each of N rows of logits (row n at logits + n*ld, V entries, dtype KD_FP32 or KD_BF16),
 * writes the K largest values and their token ids, largest first; equal values are ordered by
 * the lower token id, and -0 counts as equal to +0. Source: aiexpert.news "Making knowledge
 * distillation cheap enough to run in production", paragraph on the first fix (run the
 * teacher once, cache the 100 most probable tokens per position, reuse the cache); the
 * dailyai.com.br launch note, section "As duas inovacoes", item 1.
 *   logits [N][ld]   device, dtype (a NaN ranks below every number)
 *   idx [N][K]       device int32, written
 *   values [N][K]    device, same dtype as logits, written (copies of the selected entries)
 *   limits: 1 <= K <= min(V, 1024), V <= 4194304, ld >= V. Needs no workspace.
 * Rows of 68,272 to 204,800 bf16 (34,136 to 102,400 fp32) entries, 16-byte aligned, with
 * K <= 128 are read once, one row per compute unit at a time; other shapes, and rows whose
 * selection that pass cannot settle (NaN, many equal values, -inf), are read twice. The
 * result is the same either way.
 * The output can be passed as (idx, tlog) to the loss calls, with tlogit = dtype.
 */
kd_status kd_topk_cache(const void* logits, int32_t dtype, int64_t N, int64_t V, int64_t ld, int64_t K,
                        int32_t* idx, void* values, kd_stream stream);

/*
 * Check of a cached id table that does not synchronise: the test KD_VALIDATE_IDX runs, as two
 * kernel launches on `stream` with the result left in device memory. Every row of the cache
 * holds K distinct token ids of the vocabulary, the most probable tokens of one position
 * (aiexpert.news "Making knowledge distillation cheap enough to run in production", paragraph
 * on the first fix); this checks exactly that.
 *   idx [N][K]   device int32, read
 *   status       device, one uint32 owned by the caller: cleared by a kernel, then bit 0x1 is
 *                set if some id lies outside [0, V) and bit 0x2 if some row repeats an id.
 *   limits: 1 <= N < 2^31, 1 <= K <= 1024, V >= 1. KD_ERR_NULL if idx or status is NULL.
 * Nothing is copied to the host or waited for, so the call can be captured into a HIP graph
 * next to the loss calls; the caller reads *status once the stream has passed it. The loss
 * calls skip ids outside [0, V) without dereferencing them, and a repeated id gives wrong
 * values for its row but no fault, so a step may run before its result is read.
 */
kd_status kd_validate_ids(const int32_t* idx, int64_t N, int64_t K, int64_t V, uint32_t* status,
                          kd_stream stream);

/*
 * Per-kernel timing (profiling; off by default). While enabled, every kernel the library
 * launches, from any thread, is bracketed by two HIP events recorded on the launch's own
 * stream. kd_timing_read waits for the recorded events. It then returns, for one kernel kind,
 * the number of launches and their total duration in milliseconds accumulated since the last
 * kd_timing_reset.
 *   kd_timing_enable(on) returns the previous setting; kd_timing_kinds() is the number of
 *   kinds; kd_timing_name(kind) is a static name ("fwd", "bwd_grad", "dh", "dw", "grad_z", ...).
 * The events are owned and reused by the library; enabling timing adds two event records per
 * launch and nothing else.
 */
int kd_timing_enable(int on);
int kd_timing_kinds(void);
const char* kd_timing_name(int kind);
kd_status kd_timing_read(int kind, int64_t* launches, double* total_ms);
void kd_timing_reset(void);

#ifdef __cplusplus
}
#endif

#endif /* KDKL_H */
