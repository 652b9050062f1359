/*
 * osattn.h -- C ABI of the online-softmax attention library for AMD MI355X
 * (gfx950).  Library: online_softmax_attention_amd/libosattn.so.
 *
 * What the library computes
 * -------------------------
 * Exact scaled-dot-product attention for H independent heads:
 *
 *     s_hij  = scale * <q_hi, k_hj>
 *     O_hi   = sum_{j in A(i)} exp(s_hij - m_hi) v_hj / l_hi
 *     m_hi   = max_{j in A(i)} s_hij,   l_hi = sum_{j in A(i)} exp(s_hij - m_hi)
 *
 * (TIGA-lang "Attention and dense relations": the equations of the full
 * attention, causal dense relation and varlen causal sections.)  The admitted
 * key set A(i) is every key (dense), keys j <= i (causal), the keys of the
 * query's own sequence under cu_seqlens (varlen), or both (varlen causal).
 * The forward is one fused pass per query tile that scans key/value blocks with
 * the online-softmax recurrence: running row maximum, rescaled running sum and
 * rescaled output numerator U, with O = U / l after the last block (OCANNL
 * "Module Ir.Online_softmax", first and fourth rewrite bullets).  It never
 * materialises an (N_q, N_k) buffer.  The backward recomputes the
 * probabilities from (m, l) and uses the per-row term D_i = sum_d dO_id O_id
 * (the same page, third bullet: the fused backward).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers named q, k, v, o, d_o, dq, dk, dv, m, l, cu_seqlens and
 *    workspace are DEVICE pointers.  The caller owns all memory; the library
 *    allocates nothing and keeps no pointer after the enqueued work finishes.
 *    Outputs must not alias inputs or each other.
 *  - Tensors are 3-D (head, position, feature) with the feature index
 *    contiguous (stride 1) and element strides stride_h (between heads) and
 *    stride_n (between positions).  (H, N, D) row-major storage has
 *    stride_h = N*D, stride_n = D; (N, H, D) storage has stride_h = D,
 *    stride_n = H*D.  k and v share one stride pair; q, d_o and dq share one;
 *    dk and dv use the k/v pair; o has its own pair.
 *  - Element types: dtype OSATTN_F32, OSATTN_F16 or OSATTN_BF16 for q, k, v,
 *    d_o, dq, dk, dv.  o has o_dtype: OSATTN_F32 for any input (the default
 *    reading: the f32 accumulator divided by l, unrounded), or the input's
 *    own 16-bit type (OSATTN_F16 / OSATTN_BF16 with that input: the same f32
 *    values rounded once, to nearest even); any other o_dtype returns
 *    OSATTN_ERR_INVALID_ARG.  m and l are f32, laid out (H, n_q)
 *    contiguously; m is in natural-log units of the scaled score.
 *  - Alignment: q, k, v, d_o, dq, dk, dv, o must be 16-byte aligned and their
 *    strides multiples of 16 bytes' worth of elements (8 for f16/bf16, 4 for
 *    f32); otherwise OSATTN_ERR_ALIGNMENT.
 *  - Row strides: stride_n * element size must be <= 4 MiB for q and k/v
 *    (OSATTN_ERR_UNSUPPORTED otherwise).
 *  - Supported feature widths: d = 64 or 128, forward and backward, every
 *    dtype.  Other widths return OSATTN_ERR_UNSUPPORTED.
 *  - scale must be finite and > 0 (OSATTN_ERR_UNSUPPORTED otherwise).
 *  - causal != 0 selects j <= i; without cu_seqlens it needs n_q == n_k.
 *  - Varlen: cu_seqlens != NULL selects block-diagonal attention over
 *    num_seqs packed sequences; n_q == n_k == cu_seqlens[num_seqs] tokens and
 *    cu_seqlens holds num_seqs + 1 non-decreasing int32 values starting at 0
 *    (cumulative lengths, the flash-attn varlen convention).  max_seqlen must
 *    be >= every length (it sizes the launch grid).  The contents of
 *    cu_seqlens live on the device and are NOT checked by the library (the
 *    Python binding checks them); the kernels clamp them into [0, n_q], so
 *    malformed values give wrong results but no out-of-bounds access.
 *  - Asynchrony: work is enqueued on `stream` (a hipStream_t; NULL = the
 *    default stream) and the call returns without synchronising.  A fault in
 *    enqueued work surfaces at the caller's next synchronisation.
 *  - Errors: every entry point returns an osattn_status.  All argument checks
 *    happen on the host before any HIP call; a failed check enqueues nothing.
 *    The library never aborts, prints or throws across the ABI.
 *    osattn_last_error_message() gives a thread-local text for the last
 *    failure.  A valid call on a thread with no usable HIP device returns
 *    OSATTN_ERR_HIP (the launch fails; nothing is dereferenced on the host).
 *
 * Accuracy (fp16/bf16 inputs)
 * ---------------------------
 * The 16-bit kernels multiply in the input type with f32 accumulation.  The
 * score products and every sum are f32; the only rounding beyond f32 is that
 * of the probabilities p_ij (0 <= p <= 2^8 against the kernel's exponent
 * reference) to the input type, to nearest even, as the operand of the P.V
 * product, while l sums the unrounded f32 p.  Hence for every output row
 *
 *     |O_i - O_ref,i| <= (u + n_i t) * max_{j in A(i)} |v_j| + e32
 *
 * with u = 2^-8 (bf16) or 2^-11 (fp16), the unit roundoff of the type, n_i
 * the number of admitted keys, and t = 2^-25 for fp16 (probabilities below
 * its normal range round on a grid of 2^-24; l_i >= 1 against the kernel's
 * reference) or t = 0 for bf16 (whose range is f32's), at any scale and
 * input distribution; e32 is the error of the f32 arithmetic
 * (score sums, exponentials, row sums), below 1e-5 * max |v_j| for scores up
 * to a few hundred natural-log units.  The first term is approached only when
 * one rounding error is not averaged away, i.e. when a few keys dominate a
 * row (a sharp softmax).  On the pages' workloads -- q, k, v of unit-normal
 * size, scale <= d^-1/2 -- the error stays within the stated targets:
 * max |O - O_ref| <= 1e-2 (bf16), 2e-3 (fp16), and 1e-4 for the f32 path
 * (which rounds nothing).  Sharper softmax (scale above d^-1/2, or larger
 * |q|, |k|) moves the bf16 error toward the bound: at scale 2 d^-1/2 with
 * unit-normal inputs a randomised sweep measured 0.0122 against
 * 2^-8 * max|v| ~ 0.0176.  The backward rounds P and dS the same way as MFMA
 * operands: its error is within tol * max|ref| per gradient (tol as above)
 * on unit-normal inputs with scale <= d^-1/2, and within 2 tol * max|ref| at
 * scale 2 d^-1/2 (measured up to 1.07 tol for bf16 dQ).  m and l are f32
 * accumulations: |m - m_ref| <= 1e-4 max(1, |m_ref|) and
 * |l / l_ref - 1| <= 1e-4 on the same domain.
 */
#ifndef OSATTN_H
#define OSATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum osattn_dtype {
    OSATTN_F32 = 0,
    OSATTN_F16 = 1,
    OSATTN_BF16 = 2
} osattn_dtype;

/* Zero is success; every failure is negative. */
typedef enum osattn_status {
    OSATTN_OK = 0,
    OSATTN_ERR_INVALID_ARG = -1,  /* null pointer, bad size, bad shape */
    OSATTN_ERR_UNSUPPORTED = -2,  /* valid request this build does not serve */
    OSATTN_ERR_ALIGNMENT = -3,    /* pointer or stride not 16-byte aligned */
    OSATTN_ERR_HIP = -4,          /* the HIP runtime reported an error (also: no device) */
    OSATTN_ERR_WORKSPACE = -5     /* workspace missing or too small */
} osattn_status;

/*
 * Bytes of optional forward workspace for this problem, 0 when none is used.
 * Two cases use one:
 *  - dense relation with too few 128-row query tiles to occupy the device
 *    (fp16/bf16: and long key ranges; f32: at least 512 keys): osattn_fwd
 *    splits each tile's key range over several workgroups that write partial
 *    (m, l, U) states to the workspace, and a second kernel on the same stream
 *    combines them;
 *  - varlen (cu_seqlens given, fp16/bf16) with more than 64 sequences (up to
 *    64, each workgroup ranks its own item and no workspace is used): a
 *    first kernel writes a work list of the
 *    (sequence, query tile) items, largest first, to the workspace, and the
 *    forward takes its tiles in that order, which balances sequences of
 *    mixed lengths over the device.
 * Queries the current device's compute-unit count.  Returns 0 for invalid
 * or unsupported requests.
 */
size_t osattn_fwd_workspace_bytes(int dtype, int H, int64_t n_q, int64_t n_k, int d,
                                  int causal, const int32_t *cu_seqlens, int num_seqs,
                                  int max_seqlen);

/*
 * Forward pass.  Computes o (of o_dtype), m and l as defined above for H heads
 * of n_q queries against n_k keys of feature width d.
 *
 * workspace (device, 256-byte aligned, optional): NULL, or smaller than
 * osattn_fwd_workspace_bytes(...), runs the forward without it (unsplit, and
 * varlen tiles in their natural order); otherwise it holds the split partial
 * states or the varlen work list (contents on entry are ignored).  Results
 * are the same with or without it up to the order of the split merge (dense)
 * and bitwise the same (varlen).  Calls that share a workspace must be ordered
 * on one stream (concurrent calls race).
 *
 * Rows of o, m, l are written for every query position.  No atomics touch the
 * outputs; results are deterministic for a given problem and device.
 */
int osattn_fwd(int dtype, int o_dtype, int H, int64_t n_q, int64_t n_k, int d,
               const void *q, const void *k, const void *v,
               int64_t q_stride_h, int64_t q_stride_n,
               int64_t kv_stride_h, int64_t kv_stride_n,
               void *o, int64_t o_stride_h, int64_t o_stride_n,
               float *m, float *l,
               float scale, int causal,
               const int32_t *cu_seqlens, int num_seqs, int max_seqlen,
               void *workspace, size_t workspace_bytes,
               void *stream);

/*
 * Tile-pruned forward: an approximation of the dense forward (TIGA-lang
 * "tile-pruned sparse attention", the admission rule of its rules section).
 * Queries are cut into blocks of 128 rows and keys into tiles of 128 keys.
 * For each (head, query block) the key tiles are visited in key order with a
 * block running maximum m_run (starting at -inf): a tile whose largest
 * scaled score over all the block's rows and the tile's keys is below
 * m_run + ln(rho) is pruned -- it adds nothing to the softmax; otherwise it
 * is admitted and m_run = max(m_run, that score).  o, m, l are the exact
 * softmax results over each block's admitted keys.  The tile scores are
 * always computed; a pruned tile skips the exponentials and the P.V product.
 * Larger rho prunes more; rho = 1 keeps only tiles that reach the running
 * maximum.  There is no error bound: validate accuracy per workload.
 *
 * Dense relation only (no causal or varlen form), fp16/bf16, d = 64 or 128.
 * rho must satisfy 0 < rho <= 1 (OSATTN_ERR_INVALID_ARG otherwise; for the
 * exact result call osattn_fwd).  f32 returns OSATTN_ERR_UNSUPPORTED.
 * Arguments, layouts and errors otherwise as osattn_fwd; no workspace.
 */
int osattn_fwd_pruned(int dtype, int o_dtype, int H, int64_t n_q, int64_t n_k, int d,
                      const void *q, const void *k, const void *v,
                      int64_t q_stride_h, int64_t q_stride_n,
                      int64_t kv_stride_h, int64_t kv_stride_n,
                      void *o, int64_t o_stride_h, int64_t o_stride_n,
                      float *m, float *l, float scale, float rho,
                      void *stream);

/*
 * CSR segment softmax with given edge scores: for every head h and
 * destination row i with edges e = row_ptr[i] .. row_ptr[i+1]-1 to sources
 * col_idx[e],
 *     m_hi = max_e s_he,  l_hi = sum_e exp(s_he - m_hi),
 *     o_hi = sum_e exp(s_he - m_hi) / l_hi * v_h,col_idx[e]
 * (the relation view of TIGA-lang's attention pages -- each row's softmax
 * over its edges -- with the scores supplied as an edge field, the CSR case
 * the varlen-by-graph-composition section names for compiled streaming).
 * Dense, causal and varlen attention are special relations of this form.
 *
 * row_ptr: n_dst + 1 int32 (device), non-decreasing from 0 to nnz; col_idx:
 * nnz int32 (device) in [0, n_src); scores: f32 (H, nnz) with head stride
 * scores_stride_h (elements), finite; v: (H, n_src, d) of dtype with element
 * strides v_stride_h, v_stride_n (16-byte aligned rows); o: f32 (H, n_dst, d)
 * with its own strides; m, l: f32 (H, n_dst).  d = 64 or 128; dtype any.
 * A row with no edges gets o = 0, m = -inf, l = 0.  The CSR arrays live on
 * the device and are not checked: the kernel clamps them into range, so a
 * malformed CSR gives wrong results but no out-of-bounds access.  No
 * workspace, no atomics; asynchronous on `stream`.
 */
int osattn_csr_softmax(int dtype, int H, int64_t n_dst, int64_t n_src, int d,
                       const int32_t *row_ptr, const int32_t *col_idx, int64_t nnz,
                       const float *scores, int64_t scores_stride_h,
                       const void *v, int64_t v_stride_h, int64_t v_stride_n,
                       float *o, int64_t o_stride_h, int64_t o_stride_n,
                       float *m, float *l, void *stream);

/*
 * Bytes of device workspace osattn_bwd needs for this problem (the per-row
 * D vector and statistics, plus partial gradient sums when the launch splits
 * a reduction across workgroups).  Returns 0 for unsupported or invalid
 * requests (osattn_bwd then reports the reason).
 */
size_t osattn_bwd_workspace_bytes(int dtype, int H, int64_t n_q, int64_t n_k, int d,
                                  int causal, const int32_t *cu_seqlens, int num_seqs,
                                  int max_seqlen);

/*
 * Backward pass (OCANNL "Module Ir.Online_softmax", third bullet):
 *   D_i  = sum_d dO_id O_id
 *   P_ij = exp(s_ij - m_i) / l_i        (recomputed from q, k, m, l)
 *   dV_j = sum_i P_ij dO_i
 *   dS_ij = P_ij (<dO_i, v_j> - D_i)
 *   dQ_i = scale sum_j dS_ij k_j,   dK_j = scale sum_i dS_ij q_i
 * o, m, l are the forward's outputs for the same q, k, v, scale and mask; o
 * of o_dtype (f32, or the 16-bit input type: D_i then sums the rounded o).
 * dq uses the q strides, dk and dv the k/v strides; all are written in full,
 * in the input dtype (fp16/bf16 gradients are f32 sums rounded to nearest
 * even once at the end).
 * workspace (device, 256-byte aligned) must hold at least
 * osattn_bwd_workspace_bytes(...) bytes; its contents on entry are ignored.
 * No atomics are used: repeated calls give bit-identical gradients.
 */
int osattn_bwd(int dtype, int o_dtype, int H, int64_t n_q, int64_t n_k, int d,
               const void *q, const void *k, const void *v,
               const void *o, const void *d_o,
               int64_t q_stride_h, int64_t q_stride_n,
               int64_t kv_stride_h, int64_t kv_stride_n,
               int64_t o_stride_h, int64_t o_stride_n,
               const float *m, const float *l,
               float scale, int causal,
               const int32_t *cu_seqlens, int num_seqs, int max_seqlen,
               void *dq, void *dk, void *dv,
               void *workspace, size_t workspace_bytes,
               void *stream);

/*
 * Backward for callers that cannot allocate: code under HIP graph capture,
 * serving loops and harnesses that forbid hipMalloc.  Computes exactly what
 * osattn_bwd computes, with the same kernels and bit-identical results, but
 * takes no workspace: the library uses a static device array of
 * OSATTN_NOALLOC_SCRATCH_BYTES (32 MiB), one per GPU, held from the library's
 * load until the process ends.  Its address is looked up once per device, on
 * the first call made with that device current.  The call allocates nothing.
 *
 * Arguments, layouts and errors as osattn_bwd (without workspace and
 * workspace_bytes).  A problem whose osattn_bwd_workspace_bytes(...) exceeds
 * OSATTN_NOALLOC_SCRATCH_BYTES returns OSATTN_ERR_WORKSPACE before any HIP
 * call.  Every call on one GPU shares that GPU's array (the backward writes
 * all of it that it reads, so nothing needs clearing between calls), hence
 * calls that may overlap on one GPU -- on different streams, or from
 * different threads -- race and must be ordered by the caller.
 */
#define OSATTN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int osattn_bwd_noalloc(int dtype, int o_dtype, int H, int64_t n_q, int64_t n_k, int d,
                       const void *q, const void *k, const void *v,
                       const void *o, const void *d_o,
                       int64_t q_stride_h, int64_t q_stride_n,
                       int64_t kv_stride_h, int64_t kv_stride_n,
                       int64_t o_stride_h, int64_t o_stride_n,
                       const float *m, const float *l,
                       float scale, int causal,
                       const int32_t *cu_seqlens, int num_seqs, int max_seqlen,
                       void *dq, void *dk, void *dv,
                       void *stream);

/* Static text for a status code (never NULL). */
const char *osattn_status_string(int status);

/* Text describing the last failure on the calling thread ("" if none).  A
 * successful call clears it. */
const char *osattn_last_error_message(void);

/* Library version, as major * 10000 + minor * 100 + patch. */
int osattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* OSATTN_H */
