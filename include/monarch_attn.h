/*
 * monarch_attn.h -- C ABI of the gfx950 (MI355X) Monarch video-attention library.
 *
 * The operation (MonarchRT pages: author abstract; gist.science explainer,
 * section 2 "Methodology", parts A "Block Alignment" and B "Tiled Monarch
 * Parameterization"): attention over the N = T*H*W tokens of a video is
 * replaced by a Monarch matrix, the product of two block-diagonal factors with
 * a stride permutation between them, with blocks aligned to the video grid.
 * The factor formulas are not printed on the pages; this library fixes them:
 *
 *   tokens in (t, h, w) row-major order, n = (t*H + h)*W + w;
 *   block size b (alignment), tile tau (whole blocks, tau | N), m_tau = tau/b;
 *   token n = u*tau + i*b + j  (tile u, block i inside the tile, position j);
 *   stage 1:  Y[u,i,j] = sum_j' softmax_j'(s <Q[u,i,j], K[u,i,j']>) V[u,i,j']
 *   stage 2:  O[u,i,j] = sum_i' softmax_i'(s <Q[u,i,j], K[u,i',j]>) Y[u,i',j]
 *   s = 1/sqrt(head_dim) unless a scale is given.
 *
 * Non-causal (explainer section 2.C). Every row of every block and group has
 * at least one key, so no row is empty.
 *
 * Layout: Q, K, V, O are dense row-major [batch, heads, N, head_dim] arrays of
 * one element type (bf16 or fp32), in device memory, 16-byte aligned. The
 * stage-1 intermediate Y has the same shape and lives in a caller-provided
 * device workspace.
 *
 * Ownership: the caller owns every device buffer. A plan holds host metadata
 * only; it never allocates device memory. No entry point allocates device
 * memory or synchronises the host, and apart from monarch_attn_forward_noalloc
 * (which works in a static device array of the library) none keeps global
 * mutable state, so forwards on different streams with different workspaces may
 * run concurrently with one plan.
 *
 * Errors: every argument, plan and pointer check returns its status before any
 * HIP call, so these paths are testable on a machine without a GPU. A failed
 * kernel launch returns MONARCH_ERR_HIP. No C++ exception crosses this ABI.
 * Inf or NaN inputs are not checked; they propagate.
 */
#ifndef MONARCH_ATTN_H
#define MONARCH_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MONARCH_ABI_VERSION 5

typedef enum monarch_status {
  MONARCH_OK = 0,
  MONARCH_ERR_INVALID_ARG = 1,  /* null pointer, non-positive size, unknown enum, overflow */
  MONARCH_ERR_UNSUPPORTED = 2,  /* head_dim or dtype this build does not implement */
  MONARCH_ERR_UNALIGNED = 3,    /* b does not divide N, tile not whole blocks, split cuts a grid axis,
                                   or a device pointer not 16-byte aligned */
  MONARCH_ERR_WORKSPACE = 4,    /* workspace null or smaller than monarch_attn_workspace_size() */
  MONARCH_ERR_ALIAS = 5,        /* output overlaps an input or the workspace */
  MONARCH_ERR_HIP = 6,          /* a HIP launch failed */
  MONARCH_ERR_TOO_LARGE = 7     /* monarch_attn_forward_noalloc: the plan's workspace exceeds the
                                   library's static scratch (MONARCH_NOALLOC_SCRATCH_BYTES) */
} monarch_status;

typedef enum monarch_dtype {
  MONARCH_BF16 = 0,  /* bfloat16 storage, fp32 accumulation and softmax */
  MONARCH_FP32 = 1   /* fp32 storage and arithmetic (no reduced-precision products) */
} monarch_dtype;

/* Block alignment (explainer section 2.A): each video axis lies inside exactly one of the two
 * Monarch block dimensions. */
typedef enum monarch_align {
  MONARCH_ALIGN_FRAME = 0,   /* b = H*W: a block is one frame, a group is one (h,w) across frames */
  MONARCH_ALIGN_ROW = 1,     /* b = W: a block is one spatial row, a group is one w across (t,h) */
  MONARCH_ALIGN_DENSE = 2,   /* b = N, m = 1: ordinary softmax attention (the dense comparison) */
  MONARCH_ALIGN_TOKEN = 3,   /* b = 1, m = N: ordinary softmax attention through stage 2 alone */
  MONARCH_ALIGN_CUSTOM = 4   /* b = custom_b; must divide N; needs MONARCH_FLAG_ALLOW_UNALIGNED
                                unless b is one of W, H*W, 1, N */
} monarch_align;

#define MONARCH_FLAG_Y_FP32 (1u << 0)          /* keep Y in fp32 for bf16 inputs (default: bf16) */
#define MONARCH_FLAG_ALLOW_UNALIGNED (1u << 1) /* accept a custom b that cuts a grid axis */
#define MONARCH_FLAG_GENERIC (1u << 2)         /* force the plain VALU kernels (diagnostics) */
/* One launch for both stages (a design choice of this library; the pages describe no fused
 * two-stage kernel): the stage-1 query tiles, then the stage-2 group chunks of the same grid,
 * each chunk starting once the stage-1 blocks of its head and tile are done. Same result as the
 * two launches; on MI355X it measures slower than them. Used only where it applies (bf16, Y
 * bf16, b > 128, 2 <= m_tau <= 32: the frame and tiled alignments); elsewhere the flag is
 * ignored and monarch_plan_info.fused reports 0. It adds a control block to the workspace
 * (monarch_attn_workspace_size). */
#define MONARCH_FLAG_FUSED (1u << 3)
/* One refinement step of the Monarch factors. The pages say MonarchAttention fits its factors by
 * iterative refinement (about ten steps) and that MonarchRT needs a single step after finetuning
 * (explainer section 2.C; Spanish explainer, Resumen Ejecutivo section 2, Metodologia B); they
 * print no update equations. Reading fixed by this library: softmax attention maximises
 * F(A) = sum_r <A_r, S_r> + H(A_r) (S = s Q K^T, H the entropy) over row-stochastic A; a step
 * maximises F over the Monarch matrices one factor at a time, starting from an identity stage-2
 * factor. One step keeps stage 1 as in the direct forward (Y = R V) and refits stage 2:
 *   Kbar[u,i,j] = sum_j' R_{u,i}[j,j'] K[u,i,j']   (stage 1 applied to the keys),
 *   h[u,i,j]    = entropy (bits) of row j of R_{u,i},
 *   O[u,i,j]    = sum_i' softmax_i'(s <Q[u,i,j], Kbar[u,i',j]> + h[u,i',j] ln 2) Y[u,i',j].
 * With b = 1 or m_tau = 1 it equals the direct forward. Kbar is kept in the input dtype. The
 * workspace then holds Y, Kbar and h (monarch_attn_workspace_size). monarch_attn_forward and
 * monarch_attn_forward_noalloc compute it; monarch_attn_stage1 is unchanged (Y); stage2, chunk,
 * backward and training calls return MONARCH_ERR_UNSUPPORTED. Overrides MONARCH_FLAG_FUSED. */
#define MONARCH_FLAG_REFINE (1u << 4)

typedef struct monarch_plan monarch_plan;

typedef struct monarch_plan_info {
  int64_t batch, heads, head_dim;
  int64_t T, H, W, N;
  int64_t b;          /* block size */
  int64_t tau;        /* tile size in tokens (N when untiled) */
  int64_t m_tau;      /* blocks per tile = stage-2 group size */
  int64_t tiles;      /* U = N / tau */
  int32_t dtype;      /* monarch_dtype of Q, K, V, O */
  int32_t y_dtype;    /* monarch_dtype of the workspace Y */
  float scale;        /* softmax scale s */
  uint32_t flags;
  int64_t workspace_bytes;
  int64_t flops_stage1;  /* 4*batch*heads*N*b*head_dim (0 when stage 1 is skipped, b = 1) */
  int64_t flops_stage2;  /* 4*batch*heads*N*m_tau*head_dim (0 when stage 2 is skipped, m_tau = 1) */
  int32_t stage1_kernel; /* variant id, see monarch_attn_kernel_name() */
  int32_t stage2_kernel;
  int32_t fused;         /* 1: monarch_attn_forward makes one fused launch (MONARCH_FLAG_FUSED) */
  int32_t refine_steps;  /* 1: the forward applies one refinement step (MONARCH_FLAG_REFINE), else 0 */
  int64_t fused_error_offset; /* fused plans: byte offset in the workspace of the int32 error word
                                 (nonzero after a forward whose stage-2 wait timed out; that
                                 forward's O then holds NaN rows); -1 for other plans */
} monarch_plan_info;

/* Validate a problem and build a plan (host only, no HIP call).
 *   out          receives the plan on MONARCH_OK (else *out is set to NULL).
 *   batch, heads >= 1; head_dim in {64, 128}; T, H, W >= 1, N = T*H*W < 2^31.
 *   align        monarch_align; custom_b is read only for MONARCH_ALIGN_CUSTOM.
 *   tile_tokens  0 = untiled (tau = N); else tau, a multiple of b dividing N
 *                (explainer section 2.B: each large block cut into sub-blocks).
 *   dtype        monarch_dtype; scale 0 = 1/sqrt(head_dim), else a positive finite softmax
 *                scale (negative or non-finite: MONARCH_ERR_INVALID_ARG); flags MONARCH_FLAG_*. */
monarch_status monarch_attn_plan(monarch_plan** out, int32_t batch, int32_t heads, int32_t head_dim,
                                 int32_t T, int32_t H, int32_t W, int32_t align, int64_t custom_b,
                                 int64_t tile_tokens, int32_t dtype, float scale, uint32_t flags);

/* Free a plan (NULL is ignored). */
void monarch_attn_destroy(monarch_plan* plan);

/* Bytes of device workspace monarch_attn_forward needs (0 when b = 1 or m_tau = 1): Y, plus a
 * control block of 128 bytes plus 128 per (batch x head, tile) when the plan is fused. */
size_t monarch_attn_workspace_size(const monarch_plan* plan);

/* Copy the plan's derived sizes into *info. */
monarch_status monarch_attn_plan_info(const monarch_plan* plan, monarch_plan_info* info);

/* Full forward O = stage2(Q, K, stage1(Q, K, V)) on `stream` (a hipStream_t; NULL = default
 * stream). Asynchronous: returns after enqueueing. q, k, v, o: device pointers to
 * [batch, heads, N, head_dim] arrays of the plan's dtype. workspace: device memory of at least
 * monarch_attn_workspace_size() bytes (may be NULL when that is 0); its contents on entry are
 * ignored and on return hold Y (and the fused control block). o must not overlap q, k, v or the
 * workspace. A fused plan makes two launches (a control-block reset, then the fused kernel);
 * forwards that share one workspace must not overlap in time. When m_tau = 1 the
 * second factor is the identity and stage 1 writes O directly; when b = 1 the first factor is
 * the identity and stage 2 reads V. */
monarch_status monarch_attn_forward(const monarch_plan* plan, const void* q, const void* k,
                                    const void* v, void* o, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* The forward for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): monarch_attn_forward with the
 * workspace taken from a static device array inside the library instead of a caller argument.
 * Arguments, checks, launches and output as monarch_attn_forward; the call makes no device
 * allocation or free. The array holds MONARCH_NOALLOC_SCRATCH_BYTES bytes on every GPU the
 * library runs on, from the time the library's code is loaded there until the process ends; a
 * plan whose workspace (monarch_attn_workspace_size) is larger returns MONARCH_ERR_TOO_LARGE
 * before any HIP call. The array of the current device is used; `stream`, when not NULL, must
 * belong to the current device (else MONARCH_ERR_INVALID_ARG). All calls on one GPU share that
 * GPU's array and it keeps the last call's contents: calls that overlap in time on one GPU (on
 * different streams, or from different threads without ordering) race and give undefined
 * results. Asynchronous on `stream`. */
#define MONARCH_NOALLOC_SCRATCH_BYTES (128ll << 20)
monarch_status monarch_attn_forward_noalloc(const monarch_plan* plan, const void* q, const void* k,
                                            const void* v, void* o, void* stream);

/* Stage 1 alone (the right factor, contiguous blocks): writes Y, an array of the plan's y_dtype
 * and shape [batch, heads, N, head_dim], of y_bytes >= workspace size. When m_tau = 1 Y is the
 * final output and has the input dtype. Returns MONARCH_ERR_INVALID_ARG when b = 1 (stage 1 is
 * the identity). */
monarch_status monarch_attn_stage1(const monarch_plan* plan, const void* q, const void* k,
                                   const void* v, void* y, size_t y_bytes, void* stream);

/* Stage 2 alone (the left factor, stride-b groups inside each tile): reads Y (plan's y_dtype;
 * the input dtype when b = 1, where Y is V) and writes O. Returns MONARCH_ERR_INVALID_ARG when
 * m_tau = 1 (stage 2 is the identity). */
monarch_status monarch_attn_stage2(const monarch_plan* plan, const void* q, const void* k,
                                   const void* y, void* o, void* stream);

/* One chunk of frame-causal (autoregressive) generation: the forward for the frames
 * t0 .. t1-1 of the plan's video, where every query of the chunk sees the keys of all frames
 * before t1 (earlier chunks and the whole current chunk) - the block-causal regime of
 * autoregressive video generation the pages target (Self-Forcing, abstract). The pages give no
 * formula for it; the reading used here: stage 1 is unchanged (its blocks lie inside frames), and
 * each stage-2 group keeps its rows of frames < t1 as keys and values and its rows of frames
 * t0 .. t1-1 as queries. With t0 = 0, t1 = T it is the ordinary forward.
 *   q, k, v, o, y: [batch, heads, N, head_dim] arrays over the whole video (plan dtype; y: the
 *   plan's y_dtype). Read: q and v of frames t0..t1-1, k of frames 0..t1-1, y of frames 0..t0-1
 *   (the stage-1 outputs of earlier chunks, i.e. this call's y from earlier calls). Written: y and
 *   o of frames t0..t1-1; nothing else. y may be NULL when b = 1 (stage 1 is the identity).
 * Supported for untiled plans whose blocks lie inside frames (b divides H*W) with m_tau > 1;
 * else MONARCH_ERR_UNSUPPORTED. Asynchronous on `stream`. */
monarch_status monarch_attn_chunk_forward(const monarch_plan* plan, int32_t t0, int32_t t1, const void* q,
                                          const void* k, const void* v, void* y, void* o, void* stream);

/* Bytes of device workspace monarch_attn_backward needs (0 when the plan has no backward:
 * fp32 plans and MONARCH_FLAG_GENERIC plans). Independent of the forward's workspace. */
size_t monarch_attn_backward_workspace_size(const monarch_plan* plan);

/* Gradients of the Monarch forward (the chain rule through both softmax stages; the explainer's
 * section 2.C ships forward and backward kernels for fine-tuning): given O = forward(Q, K, V)
 * and grad_o = dL/dO, writes grad_q = dL/dQ, grad_k = dL/dK, grad_v = dL/dV. All nine arrays are
 * [batch, heads, N, head_dim] bf16 device arrays (bf16 plans only; fp32 plans return
 * MONARCH_ERR_UNSUPPORTED); o must be the output of monarch_attn_forward for the same inputs.
 * Stage 1 is recomputed (its output Y and per-row softmax statistics go to the workspace, whose
 * contents on entry are ignored; a plan whose only stage has at most 128 rows per problem skips
 * it), then the stage-2 backward and the stage-1 backward run, fp32 accumulation throughout;
 * stages with at most 128 rows per problem recompute their softmax statistics inside their
 * one-pass backward. Q and K receive the sum of both stages' gradients. grad_* must
 * not overlap each other, the inputs or the workspace. Asynchronous on `stream`. */
monarch_status monarch_attn_backward(const monarch_plan* plan, const void* q, const void* k, const void* v,
                                     const void* o, const void* grad_o, void* grad_q, void* grad_k,
                                     void* grad_v, void* workspace, size_t workspace_bytes, void* stream);

/* Training forward: writes O = forward(Q, K, V) like monarch_attn_forward and leaves in
 * `workspace` (a backward workspace: monarch_attn_backward_workspace_size bytes) the state the
 * backward would otherwise recompute: the stage-1 output Y (bf16) and stage 1's per-row softmax
 * statistics. The launches are those of the backward's recompute followed by stage 2, always the
 * two-launch path with bf16 Y; for plans without MONARCH_FLAG_Y_FP32 and MONARCH_FLAG_FUSED, O
 * is bitwise the output of monarch_attn_forward. bf16 plans with a backward only (else
 * MONARCH_ERR_UNSUPPORTED); o must not overlap the inputs or the workspace, nor the workspace
 * the inputs. Asynchronous on `stream`. */
monarch_status monarch_attn_forward_train(const monarch_plan* plan, const void* q, const void* k, const void* v,
                                          void* o, void* workspace, size_t workspace_bytes, void* stream);

/* monarch_attn_backward without the forward recompute: `workspace` must hold the state a
 * monarch_attn_forward_train call with the same plan, q, k and v left there, unchanged since
 * (any other backward call on it overwrites that state). Arguments, checks, errors and outputs
 * as monarch_attn_backward; with such a workspace the gradients are bitwise those of
 * monarch_attn_backward. With any other workspace contents the call still returns MONARCH_OK
 * and touches no memory outside its arguments, but the gradients are meaningless. */
monarch_status monarch_attn_backward_saved(const monarch_plan* plan, const void* q, const void* k, const void* v,
                                           const void* o, const void* grad_o, void* grad_q, void* grad_k,
                                           void* grad_v, void* workspace, size_t workspace_bytes, void* stream);

/* Static description of a status code (never NULL; "unknown status" for a value
 * that is no monarch_status). The code is taken as a plain integer so that any
 * value is well defined to pass. */
const char* monarch_status_string(int32_t status);

/* Static name of a kernel variant id from monarch_plan_info (never NULL). */
const char* monarch_attn_kernel_name(int32_t kernel_id);

/* MONARCH_ABI_VERSION of the loaded library. */
int32_t monarch_attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MONARCH_ATTN_H */
