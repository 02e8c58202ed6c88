/*
 * lora_mi355x.h -- C ABI of the fused LoRA / QLoRA projection library for
 * AMD Instinct MI355X (CDNA4, gfx950).
 *
 * The library computes the data-parallel hot path of LoRA fine-tuning of a
 * transformer block: the gated LoRA MLP (gate, up and down projections around
 * a SwiGLU or GeGLU activation), the LoRA Q/K/V projections and the single
 * LoRA projection used for the attention output (O), forward and backward,
 * with an optional NF4-packed frozen base weight.
 *
 * Sources the operations follow (cited by page title and section):
 *   [LO]  "LoRA Optimizations" -- Axolotl documentation: sections "Custom
 *         autograd functions", "Triton kernels", "Integration", "Requirements".
 *   [UD]  unsloth compare view main...fix/fused-lora-fp32-dtype: the commit
 *         message "Avoid recomputing LoRA B-projected gradient in fused-LoRA
 *         backward" and the hunks of LoRA_MLP, LoRA_QKV, LoRA_W, matmul_lora.
 *   [LL]  "loralei" README: section "Use", QLoRA paragraphs (NF4 block sizes,
 *         fused unpack and double-scale reconstruction inside the matmul).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout.  Every matrix is row-major and densely packed (leading dimension =
 *   number of columns).  A LoRA projection maps width n_in to n_out and has a
 *   frozen base W [n_in, n_out], adapters A [n_in, r] and B [r, n_out] and a
 *   scale s (alpha/r, or alpha/sqrt(r), the caller's choice):
 *       U = X A          Z = X W + s (U B)                          ([UD] LoRA_W)
 *   Gradients dA, dB have the layout of A, B.
 * Memory.  All tensor pointers are device memory owned by the caller; the
 *   library never allocates or frees device memory, and no call's result
 *   depends on an earlier call.  The only state it holds: the calling
 *   thread's last error text (lora_last_error), the tracing records (off by
 *   default; see lora_trace_begin) and, for lora_o_fwd_noalloc only, the
 *   address of each GPU's static scratch array.
 *   Scratch memory comes from the caller's workspace (ws, ws_bytes), whose
 *   minimum size the matching *_workspace_size query returns.  Descriptor
 *   structs (lora_*_desc, lora_proj, lora_nf4, lora_*_grads) live in host
 *   memory and are read during the call only.
 * dtype.  One compute dtype per call: LORA_BF16 (bf16 in and out, fp32
 *   accumulation) or LORA_F32 (fp32 throughout).  Every dense tensor of the
 *   call (X, W, A, B, outputs, saved tensors) has that dtype.  NF4 bases need
 *   bf16 compute (LORA_BF16 or LORA_BF16_F32LORA).
 *   LORA_BF16_F32LORA is the fp32 LoRA-gradient mode ([LO] "FP32 LoRA
 *   gradients"): the adapters A, B and the gradients dA, dB are fp32; every
 *   other tensor (X, W, dY, outputs, saved e, g, U, dX) is bf16.  Each call
 *   first casts A and B to bf16 (round to nearest even) into its workspace and
 *   runs the bf16 path on the casts; dA and dB are the fp32 sums of the bf16
 *   products, times s, stored without the final rounding to bf16.  The
 *   rank-r intermediates (U, P) stay bf16, as in LORA_BF16.
 * Streams.  `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *   enqueue work on it and return; inputs are read-only; results are ready
 *   when the stream reaches them.  Calls on distinct streams with distinct
 *   buffers may run concurrently.
 * Errors.  Arguments are validated on the host before anything is enqueued;
 *   on any error the call returns a lora_status other than LORA_OK, enqueues
 *   nothing and writes nothing.  A launch failure reported by the HIP runtime
 *   after enqueue returns LORA_EDEVICE.  lora_last_error() gives a text detail
 *   of the calling thread's last failure.
 * Shapes (both bf16 modes).  T >= 0 is any token count (T = 0 is a no-op that still
 *   zero-fills adapter gradients).  Feature widths (H, I, Nq, Nk, Nv, K, N)
 *   must be positive multiples of 64 and r a multiple of 8 in [8, 64], with
 *   the concatenated adapter width of a shared-input group (2r for gate/up,
 *   3r for Q/K/V) at most 64.  Pointers must be 16-byte aligned.
 * Shapes (fp32).  Any positive widths, 1 <= r <= 64; 4-byte aligned pointers.
 * Extent (all dtypes).  The kernels address each operand with 32-bit byte
 *   offsets: every activation [T, width] and every weight must be smaller
 *   than 2 GiB - 4 KiB, else the call returns LORA_ESHAPE.
 * No dropout and no bias on the adapters ([LO] "Requirements").
 */
#ifndef LORA_MI355X_H
#define LORA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LORA_MI355X_VERSION 3

typedef enum lora_status {
  LORA_OK = 0,
  LORA_EINVAL = 1,       /* null pointer, unknown enum, negative size */
  LORA_ESHAPE = 2,       /* shape not supported (see "Shapes" above) */
  LORA_EDTYPE = 3,       /* unknown or mismatched dtype */
  LORA_EALIGN = 4,       /* pointer not aligned as required */
  LORA_EWORKSPACE = 5,   /* ws missing or smaller than the query's size */
  LORA_EUNSUPPORTED = 6, /* valid but unsupported (NF4 with fp32, partial aliasing) */
  LORA_EDEVICE = 7       /* HIP runtime reported an error */
} lora_status;

typedef enum lora_dtype { LORA_F32 = 0, LORA_BF16 = 1, LORA_BF16_F32LORA = 2 } lora_dtype;

/* Gated activation phi of h = phi(e) * g ([LO] "Triton kernels"):
 *   SWIGLU:      phi(x) = x * sigmoid(x)
 *   GEGLU_TANH:  phi(x) = x/2 * (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))   */
typedef enum lora_act { LORA_ACT_SWIGLU = 0, LORA_ACT_GEGLU_TANH = 1 } lora_act;

/* NF4-packed frozen base weight W [rows, cols] = [n_in, n_out] ([LL] "Use",
 * QLoRA paragraphs).  Arrays are device memory, written by lora_nf4_quantize.
 *   codes: numel/2 bytes; byte j holds the code of element 2j in bits 7..4 and
 *          of element 2j+1 in bits 3..0 (elements in row-major order);
 *   q8:    numel/64 int8, one per block of 64 consecutive elements;
 *   s2:    numel/16384 float, one per scaler block of 256 blocks;
 *   mu:    one float (mean block absmax).
 * Element j of block b of scaler block S dequantizes to
 *   a'  = fl32(fl32(q8[b] * s2[S]) + mu)
 *   w'  = fl32(c[code_j] * a')          (bf16 form: w' rounded to nearest even)
 * with c the 16 NF4 levels of the QLoRA paper (see lora_nf4_codebook).
 * rows * cols must be a multiple of 64 * 256. */
typedef struct lora_nf4 {
  const uint8_t* codes;
  const int8_t* q8;
  const float* s2;
  const float* mu;
  int64_t rows;
  int64_t cols;
} lora_nf4;

/* One LoRA projection: exactly one of W (dense, compute dtype) and nf4 is
 * non-NULL.  A [n_in, r], B [r, n_out] in the compute dtype (fp32 under
 * LORA_BF16_F32LORA); scale = s.
 * Wt (optional, dense bf16 only, else NULL): the same frozen weight stored
 * [n_out, n_in], i.e. W^T, PyTorch nn.Linear's own layout.  The forward
 * product X W reads the weight along n_in; from Wt that is a K-contiguous
 * operand, which the bf16 GEMM loads and feeds to the matrix cores with
 * fewer LDS reads than W's N-contiguous rows.  When every projection of a
 * forward GEMM has Wt (gate and up together, q, k and v together), that GEMM
 * reads Wt; backward GEMMs always read W.  Wt must hold exactly W^T (not
 * checked); it is ignored in fp32. */
typedef struct lora_proj {
  const void* W;
  const lora_nf4* nf4;
  const void* A;
  const void* B;
  float scale;
  const void* Wt;
} lora_proj;

/* Optional launch plan of a call's GEMMs ("loralei" README, section "Use":
 * per GPU and shape, a few valid tile configurations are timed and the
 * fastest is kept in a cache, with a conservative default on a miss).  The
 * library keeps no such cache: a caller (the Python tuner in
 * adapter_mlp_amd.tune) times candidates, stores the winners, and passes the
 * plan for a shape in the call's descriptor; NULL, or an all-zero entry,
 * keeps the library's defaults.  Plans change only the order of work and
 * how K is split, never what is computed; they are ignored in fp32.
 *   group:  m-tiles per group of the XCD-aware tile order (the tiles an XCD
 *           holds at once share group activation panels): 0 = default (4 for
 *           activation epilogues, 8 for plain stores), or 1, 2, 4, 8, 16, 32;
 *   ksplit: 0 = the library's split-K model, 1 = no split, 2..4 = that many
 *           K parts (fp32 partials in the workspace, added in a fixed order).
 *           Only a dense plain-store GEMM with one output region can split;
 *           elsewhere ksplit must be 0 or 1.  Each part needs at least one
 *           K step of 64.  When the 256x256 tiles fill one or more whole
 *           rounds of 256 CUs, only the tiles left over are split (the same
 *           number of rounds as splitting all, with fewer partial sums).
 * gemm[] lists the call's GEMMs in launch order: gated / ReLU^2 MLP forward:
 * [0] gate/up (or up), [1] down; MLP backward: [0] dh, [1] dX; Q/K/V and O,
 * forward or backward: [0] (gemm[1] must be zero).  An invalid entry returns
 * LORA_EINVAL.  The workspace queries take the plan into account. */
typedef struct lora_gemm_plan {
  int32_t group;
  int32_t ksplit;
} lora_gemm_plan;

typedef struct lora_plan {
  lora_gemm_plan gemm[2];
} lora_plan;

/* ------------------------------------------------------------------------ */
/* Library information                                                       */
/* ------------------------------------------------------------------------ */

int lora_version(void);
const char* lora_strerror(lora_status status);
/* Text detail of the calling thread's last non-OK status (never NULL). */
const char* lora_last_error(void);
/* Copies the library's 16 NF4 levels (float32, ascending) to host out[16]. */
void lora_nf4_codebook(float* out);

/* ------------------------------------------------------------------------ */
/* Gated LoRA MLP block ([UD] LoRA_MLP; [LO] "Custom autograd functions")     */
/* ------------------------------------------------------------------------ */

typedef struct lora_mlp_desc {
  int64_t T;     /* tokens (rows of X) */
  int64_t H;     /* hidden size (width of X and Y) */
  int64_t I;     /* intermediate size (width of e, g, h) */
  int64_t r;     /* adapter rank, shared by gate, up and down */
  int32_t act;   /* lora_act */
  int32_t dtype; /* lora_dtype */
  const lora_plan* plan; /* optional GEMM launch plan (NULL: defaults) */
} lora_mlp_desc;

/* Tensors the forward saves for the backward (caller-owned, compute dtype):
 *   e [T, I] = gate projection, g [T, I] = up projection,
 *   U [T, 3r] = [X A_gate | X A_up | h A_down] (unscaled adapter inputs). */
typedef struct lora_mlp_saved {
  void* e;
  void* g;
  void* U;
} lora_mlp_saved;

/* Adapter gradients written by the backward (each the layout and dtype of its
 * A/B). */
typedef struct lora_mlp_grads {
  void* dA_gate;
  void* dB_gate;
  void* dA_up;
  void* dB_up;
  void* dA_down;
  void* dB_down;
} lora_mlp_grads;

/* Minimum workspace sizes of lora_mlp_fwd and lora_mlp_bwd for `desc`. */
lora_status lora_mlp_workspace_size(const lora_mlp_desc* desc, size_t* fwd_bytes,
                                    size_t* bwd_bytes);

/* Forward:  e = Z_gate(X), g = Z_up(X), h = phi(e) * g, Y = Z_down(h), each Z a
 * LoRA projection.  In bf16, e and g are rounded to bf16 and h is formed from
 * the rounded values (the backward recomputes h bit for bit).
 * X [T, H] -> Y [T, H]; writes saved->e, saved->g, saved->U. */
lora_status lora_mlp_fwd(const lora_mlp_desc* desc, const void* X, const lora_proj* gate,
                         const lora_proj* up, const lora_proj* down, void* Y,
                         const lora_mlp_saved* saved, void* ws, size_t ws_bytes,
                         void* stream);

/* Backward, given dY [T, H] and the forward's X and saved tensors:
 *   P_d = dY B_d^T (formed once), dh = dY W_d^T + s_d P_d A_d^T,
 *   dA_d = s_d h^T P_d, dB_d = s_d U_d^T dY,
 *   dg = dh * phi(e), de = dh * g * phi'(e),
 *   P_u = dg B_u^T, P_g = de B_g^T (each formed once and used twice),
 *   dA_u = s_u X^T P_u, dB_u = s_u U_u^T dg, dA_g = s_g X^T P_g, dB_g = s_g U_g^T de,
 *   dX = dg W_u^T + s_u P_u A_u^T + de W_g^T + s_g P_g A_g^T.
 * Outputs are overwritten (not accumulated).  dX may be X itself
 * (in place: X is last read by the dA pass, which precedes the dX GEMM); a
 * partial overlap of dX and X is rejected (LORA_EUNSUPPORTED). */
lora_status lora_mlp_bwd(const lora_mlp_desc* desc, const void* dY, const void* X,
                         const lora_mlp_saved* saved, const lora_proj* gate,
                         const lora_proj* up, const lora_proj* down, void* dX,
                         const lora_mlp_grads* grads, void* ws, size_t ws_bytes,
                         void* stream);

/* ------------------------------------------------------------------------ */
/* Ungated ReLU^2 LoRA MLP ([LO] "FP32 LoRA gradients": the dense ReLU^2     */
/* MLPs of Nemotron-H, up and down LoRA projections with a fused ReLU^2      */
/* activation derivative)                                                    */
/* ------------------------------------------------------------------------ */

typedef struct lora_relu2_mlp_desc {
  int64_t T;        /* tokens */
  int64_t H;        /* hidden size (width of X and Y) */
  int64_t I;        /* intermediate size (width of u and h) */
  int64_t r;        /* adapter rank, shared by up and down */
  int32_t dtype;    /* lora_dtype */
  int32_t reserved; /* must be 0 */
  const lora_plan* plan; /* optional GEMM launch plan (NULL: defaults) */
} lora_relu2_mlp_desc;

/* Saved by the forward (caller-owned, compute dtype): u [T, I] = the up
 * projection; U [T, 2r] = [X A_up | h A_down] (unscaled adapter inputs). */
typedef struct lora_relu2_mlp_saved {
  void* u;
  void* U;
} lora_relu2_mlp_saved;

typedef struct lora_relu2_mlp_grads {
  void* dA_up;
  void* dB_up;
  void* dA_down;
  void* dB_down;
} lora_relu2_mlp_grads;

lora_status lora_relu2_mlp_workspace_size(const lora_relu2_mlp_desc* desc, size_t* fwd_bytes,
                                          size_t* bwd_bytes);

/* Forward:  u = Z_up(X), h = max(u, 0)^2, Y = Z_down(h).  In bf16, u is
 * rounded to bf16 and h is formed from the rounded u (the backward recomputes
 * h bit for bit).  X [T, H] -> Y [T, H]; writes saved->u, saved->U.  The bf16
 * rank limit is r <= 64. */
lora_status lora_relu2_mlp_fwd(const lora_relu2_mlp_desc* desc, const void* X, const lora_proj* up,
                               const lora_proj* down, void* Y, const lora_relu2_mlp_saved* saved, void* ws,
                               size_t ws_bytes, void* stream);

/* Backward, given dY [T, H] and the forward's X and saved tensors:
 *   P_d = dY B_d^T (formed once), dh = dY W_d^T + s_d P_d A_d^T,
 *   dA_d = s_d h^T P_d, dB_d = s_d U_d^T dY, du = dh * 2 max(u, 0),
 *   P_u = du B_u^T (formed once), dA_u = s_u X^T P_u, dB_u = s_u U_u^T du,
 *   dX = du W_u^T + s_u P_u A_u^T.
 * Outputs are overwritten.  dX may be X itself
 * (in place: X is last read by the dA pass, which precedes the dX GEMM); a
 * partial overlap of dX and X is rejected (LORA_EUNSUPPORTED). */
lora_status lora_relu2_mlp_bwd(const lora_relu2_mlp_desc* desc, const void* dY, const void* X,
                               const lora_relu2_mlp_saved* saved, const lora_proj* up, const lora_proj* down,
                               void* dX, const lora_relu2_mlp_grads* grads, void* ws, size_t ws_bytes,
                               void* stream);

/* ------------------------------------------------------------------------ */
/* LoRA Q/K/V projections of one input ([UD] LoRA_QKV; [LO] attention       */
/* patch: apply_qkv)                                                         */
/* ------------------------------------------------------------------------ */

typedef struct lora_qkv_desc {
  int64_t T, H;       /* tokens, input width */
  int64_t Nq, Nk, Nv; /* output widths of Q, K, V */
  int64_t r;          /* adapter rank shared by q, k, v */
  int32_t dtype;
  int32_t reserved;   /* must be 0 */
  const lora_plan* plan; /* optional GEMM launch plan (NULL: defaults) */
} lora_qkv_desc;

typedef struct lora_qkv_grads {
  void* dA_q;
  void* dB_q;
  void* dA_k;
  void* dB_k;
  void* dA_v;
  void* dB_v;
} lora_qkv_grads;

lora_status lora_qkv_workspace_size(const lora_qkv_desc* desc, size_t* fwd_bytes,
                                    size_t* bwd_bytes);

/* Q = Z_q(X) [T, Nq], K = Z_k(X) [T, Nk], V = Z_v(X) [T, Nv];
 * U [T, 3r] = [X A_q | X A_k | X A_v] saved for the backward. */
lora_status lora_qkv_fwd(const lora_qkv_desc* desc, const void* X, const lora_proj* q,
                         const lora_proj* k, const lora_proj* v, void* Q, void* K, void* V,
                         void* U, void* ws, size_t ws_bytes, void* stream);

/* dX = sum over p in {q,k,v} of (dZ_p W_p^T + s_p P_p A_p^T) with P_p = dZ_p B_p^T
 * formed once; dA_p = s_p X^T P_p; dB_p = s_p U_p^T dZ_p.  dX may be X itself
 * (in place: X is last read by the dA pass, which precedes the dX GEMM); a
 * partial overlap of dX and X is rejected (LORA_EUNSUPPORTED). */
lora_status lora_qkv_bwd(const lora_qkv_desc* desc, const void* dQ, const void* dK,
                         const void* dV, const void* X, const void* U, const lora_proj* q,
                         const lora_proj* k, const lora_proj* v, void* dX,
                         const lora_qkv_grads* grads, void* ws, size_t ws_bytes,
                         void* stream);

/* ------------------------------------------------------------------------ */
/* Single LoRA projection, used for O ([UD] LoRA_W, apply_lora_o)            */
/* ------------------------------------------------------------------------ */

typedef struct lora_o_desc {
  int64_t T;   /* tokens */
  int64_t K;   /* input width n_in */
  int64_t N;   /* output width n_out */
  int64_t r;
  int32_t dtype;
  int32_t reserved; /* must be 0 */
  const lora_plan* plan; /* optional GEMM launch plan (NULL: defaults) */
} lora_o_desc;

lora_status lora_o_workspace_size(const lora_o_desc* desc, size_t* fwd_bytes,
                                  size_t* bwd_bytes);

/* Y [T, N] = X W + s (X A) B; U [T, r] = X A saved. */
lora_status lora_o_fwd(const lora_o_desc* desc, const void* X, const lora_proj* o, void* Y,
                       void* U, void* ws, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the forward
 * of lora_o_fwd with no workspace argument.  The call allocates nothing; its
 * scratch is a static device array of LORA_NOALLOC_SCRATCH_BYTES per GPU,
 * part of the library's code object, held until the process ends, and looked
 * up on the calling thread's current device (which must be the device of the
 * buffers and of `stream`) at that device's first call.  The caller passes
 * inputs and outputs as for lora_o_fwd, with the same results; the GEMM never
 * uses split-K here.  A call whose scratch need exceeds the limit (about
 * 128 bytes per token plus 128 bytes per output column and 2 r K bytes in
 * bf16; the fp32 adapter casts add 2 r (K + N) bytes under LORA_BF16_F32LORA;
 * 4 r (T + N + K) bytes in fp32)
 * returns LORA_EWORKSPACE and enqueues nothing.  Every call on one GPU uses
 * the same array: calls that can overlap on one GPU (on different streams,
 * or from different threads) race and must be ordered by the caller.
 * LORA_EDEVICE if the array's address cannot be obtained. */
#define LORA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
lora_status lora_o_fwd_noalloc(const lora_o_desc* desc, const void* X, const lora_proj* o, void* Y, void* U,
                               void* stream);

/* P = dY B^T (once); dX = dY W^T + s P A^T; dA = s X^T P; dB = s U^T dY.
 * dX may be X itself (in place); a partial overlap is rejected. */
lora_status lora_o_bwd(const lora_o_desc* desc, const void* dY, const void* X, const void* U,
                       const lora_proj* o, void* dX, void* dA, void* dB, void* ws,
                       size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* NF4 format ([LL] "Use", QLoRA paragraphs)                                 */
/* ------------------------------------------------------------------------ */

/* Workspace for lora_nf4_quantize of a [rows, cols] weight. */
lora_status lora_nf4_quantize_workspace_size(int64_t rows, int64_t cols, size_t* bytes);

/* Quantize W [rows, cols] (device, dtype LORA_F32 or LORA_BF16) to NF4:
 *   block absmax a_b = max |w| over 64 consecutive elements;
 *   code = nearest level to fl32(w / a_b) (ties to the lower level; a_b = 0 -> level 0.0);
 *   mu = fl32(S / nblocks), S the fp64 sum of a_b taken per scaler block in
 *        ascending order, then over scaler blocks in ascending order;
 *   per scaler block: d_b = fl32(a_b - mu), s2 = fl32(max|d_b| / 127),
 *        q8_b = clamp(rint(fl32(d_b / s2)), -127, 127), or 0 when s2 = 0.
 * Outputs: codes [numel/2], q8 [numel/64], s2 [numel/16384], mu [1] (device). */
lora_status lora_nf4_quantize(const void* W, int64_t rows, int64_t cols, int32_t dtype,
                              uint8_t* codes, int8_t* q8, float* s2, float* mu, void* ws,
                              size_t ws_bytes, void* stream);

/* out [rows, cols] = dequantized weight, float32 (LORA_F32) or bf16 (LORA_BF16). */
lora_status lora_nf4_dequant(const lora_nf4* w, void* out, int32_t dtype, void* stream);

/* out [rows * cols] = the 4-bit code of every element, one byte each. */
lora_status lora_nf4_unpack_codes(const lora_nf4* w, uint8_t* out, void* stream);

lora_status lora_nf4_gemm_workspace_size(int64_t T, int64_t rows, int64_t cols, int64_t r,
                                         int32_t trans, size_t* bytes);

/* Dequant-GEMM with the NF4 unpack and scale reconstruction done in registers
 * inside the matmul ([LL] "Use": fused forward and input-gradient matmuls).
 *   trans = 0 (forward):         Y [T, cols] = X [T, rows] deq(W) + s (X A) B
 *   trans = 1 (input gradient):  Y [T, rows] = X [T, cols] deq(W)^T + s (X B^T) A^T
 * A [rows, r] and B [r, cols] (bf16) may both be NULL (r ignored) for the plain
 * product.  bf16 only. */
lora_status lora_nf4_gemm(int64_t T, int32_t trans, const void* X, const lora_nf4* W,
                          const void* A, const void* B, int64_t r, float scale, void* Y,
                          void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Kernel timing (tracing)                                                   */
/* ------------------------------------------------------------------------ */

/* Per-kernel totals of the launches recorded between lora_trace_begin and
 * lora_trace_end.  While tracing is on, every kernel the library enqueues is
 * bracketed by two HIP events recorded on its launch stream; the pair's
 * elapsed time is that launch's duration.  Tracing is process-wide state and
 * is off by default.  While it is off a launch only reads one atomic flag;
 * while it is on each launch adds two event records and takes one
 * process-wide lock (a debugging and measurement aid, not for production). */
typedef struct lora_trace_entry {
  char name[48];     /* kernel family, e.g. "gemm_nn_act_fwd" */
  int64_t launches;
  double total_ms;
} lora_trace_entry;

/* Start recording (clears earlier records).  `prefix` limits recording to
 * kernel families whose name starts with it (NULL or "" records all). */
lora_status lora_trace_begin(const char* prefix);

/* Stop recording, wait for the recorded events, and write up to `max` entries
 * (one per kernel family, in first-launch order) to out; *count receives the
 * number of families.  LORA_EDEVICE if an event could not be read. */
lora_status lora_trace_end(lora_trace_entry* out, int32_t max, int32_t* count);

#ifdef __cplusplus
}
#endif

#endif /* LORA_MI355X_H */
