/*
 * qlora.h - C ABI of the MI355X (gfx950) QLoRA linear / gated-MLP library.
 *
 * What is computed (the pages' statement of the problem):
 *   - Frozen base weights W are stored in 4-bit NormalFloat ("QLoRA nf4" on
 *     q/k/v/o/gate/up/down; Mistral benchmark page, configuration block) and
 *     dequantized to bfloat16, never to float16 (same page, breakdown item 2,
 *     "Bitsandbytes bfloat16").
 *   - A rank-r LoRA side path with scale s = alpha / r (rank 16, alpha 16,
 *     dropout 0 in the configuration block), bracketed rank-first:
 *     X A^T is formed before anything of width in x out; the merged weight
 *     W + s B A is never formed (same page, items 10-11 "manual autograd",
 *     chained-matmul bracketing).
 *   - Hand-derived backward producing dX, dA, dB; no gradient of the frozen W
 *     (Show HN thread: "manual autograd engine - hand derived backprop").
 *   - Gated MLP gate/up -> act -> down with SwiGLU (silu(g) * u) or tanh-GeGLU
 *     (gelu_tanh(g) * u) (Gemma page, "GeGLU vs SwiGLU activation"), whose
 *     activation is recomputed in the backward rather than stored.
 *
 * Conventions (all entry points):
 *   - Every tensor pointer is a DEVICE pointer unless stated otherwise.
 *     Tensors are row-major and dense (leading dimension = row length).
 *   - bf16 tensors are passed as uint16_t bit patterns.
 *   - NF4 weight of shape [n][k]: codes uint8 [n][k/2], element 2j of a row in
 *     the HIGH nibble of byte j and element 2j+1 in the LOW nibble; absmax
 *     float32 [n][k/64], one per 64 consecutive weights of a row. Dequantized
 *     value: bf16_rne(fp32_rne(level[code] * absmax)).
 *   - LoRA factors: A [r][in], B [out][r], bf16.
 *   - `stream` is a hipStream_t (NULL = the null stream). Every call only
 *     enqueues work on it and returns; nothing synchronizes the host.
 *   - The library never allocates device memory. Scratch space is the
 *     caller's `ws` buffer of at least the size returned by the matching
 *     *_workspace_bytes() query (any 256-byte aligned device allocation).
 *   - Validation errors return before anything is enqueued. A HIP launch
 *     failure returns QLORA_EHIP; qlora_last_error() then gives the HIP
 *     message (per thread).
 *   - Shape limits: k, n (and d, h) multiples of 64; m >= 0; 1 <= r <= 64
 *     (the pages call 16 and 64 the usual ranks; Mistral benchmark page,
 *     items 10-11). m == 0 writes only the LoRA gradients (as zeros); the
 *     per-token tensors may then be NULL. Output buffers must not alias
 *     inputs.
 *   - Alignment: every bf16 matrix (X, Y, dY, dX, g, u, 16-bit base weights,
 *     LoRA factors A and B) and every NF4 code array starts on a 16-byte
 *     boundary; absmax and the fp32 U / T tensors on 4 bytes; the bf16 LoRA
 *     gradients dA, dB on 2 bytes. A pointer off its boundary returns
 *     QLORA_ESHAPE before anything is enqueued (device allocations and
 *     contiguous tensors at offset 0 always qualify).
 *   - Results are deterministic: two identical calls give identical bits
 *     (no floating-point atomics; fixed reduction order).
 *   - Calls that share one workspace buffer must not overlap in time.
 */
#ifndef QLORA_H
#define QLORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QLORA_OK = 0,
  QLORA_EINVAL = -1,     /* null pointer, bad r, non-finite s, unknown act/flag */
  QLORA_ESHAPE = -2,     /* k or n not a multiple of 64, negative m, size overflow */
  QLORA_EWORKSPACE = -3, /* ws NULL or ws_bytes below the query's answer */
  QLORA_EHIP = -4,       /* HIP launch/runtime error (including no device) */
  QLORA_ENOTIMPL = -5    /* valid request that this library does not implement */
} qlora_status;

typedef enum { QLORA_ACT_SWIGLU = 0, QLORA_ACT_GEGLU_TANH = 1 } qlora_act;

/* How the NF4 base weight reaches the bf16 matrix cores.
 *   QLORA_DEQUANT_AUTO   : the library's measured default for the shape.
 *   QLORA_DEQUANT_FUSED  : codes are dequantized inside the GEMM while the
 *                          weight tile is staged into LDS (no bf16 copy).
 *   QLORA_DEQUANT_STAGED : each weight is first dequantized once into the
 *                          workspace, then a plain bf16 GEMM reads it.
 * Both give the same dequantized weights; results agree to rounding order. */
typedef enum {
  QLORA_DEQUANT_AUTO = 0,
  QLORA_DEQUANT_FUSED = 1,
  QLORA_DEQUANT_STAGED = 2
} qlora_dequant_mode;

/* An NF4-quantized weight of shape [n][k] (device pointers).
 * Its per-block constants are either the fp32 absmax array, or (absmax NULL)
 * that array double-quantized by qlora_absmax_dq_quantize: one int8 code per
 * 64-weight block and one fp32 scale and offset per 256 consecutive blocks
 * (flattened row-major), absmax[i] = fp32(fp32(q[i] * scale[i/256]) +
 * offset[i/256]). Every entry point that takes a qlora_nf4 accepts both forms
 * and dequantizes with the reconstructed absmax; the trailing fields may stay
 * zero (NULL) for a plain weight. The QLoRA paper, which the pages link for
 * the 4-bit format, stores its constants this way ("double quantization"). */
typedef struct qlora_nf4 {
  const uint8_t* codes;        /* [n][k/2] */
  const float* absmax;         /* [n][k/64], or NULL when double-quantized */
  int64_t n;
  int64_t k;
  const int8_t* absmax_q;      /* [n*k/64] codes (double-quantized form) */
  const float* absmax_scale;   /* [ceil(n*k/64 / 256)] */
  const float* absmax_offset;  /* [ceil(n*k/64 / 256)] */
} qlora_nf4;

/* The three projections of a gated MLP with hidden width d and MLP width h
 * (Llama/Mistral/Gemma layout): gate, up [h][d]; down [d][h]; LoRA factors
 * A_gate, A_up [r][d], B_gate, B_up [h][r], A_down [r][h], B_down [d][r].
 * Passed by HOST pointer; the pointers inside are device pointers. */
typedef struct qlora_mlp_weights {
  qlora_nf4 gate, up, down;
  const uint16_t* a_gate;
  const uint16_t* b_gate;
  const uint16_t* a_up;
  const uint16_t* b_up;
  const uint16_t* a_down;
  const uint16_t* b_down;
  int64_t d, h, r;
  float s;   /* LoRA scale alpha / r (or any finite scale, e.g. rank-stabilised) */
  int act;   /* qlora_act */
} qlora_mlp_weights;

/* LoRA weight gradients of the MLP (device pointers, bf16, same shapes as
 * the factors). Passed by HOST pointer. */
typedef struct qlora_mlp_grads {
  uint16_t* a_gate;
  uint16_t* b_gate;
  uint16_t* a_up;
  uint16_t* b_up;
  uint16_t* a_down;
  uint16_t* b_down;
} qlora_mlp_grads;

/* Text for a status code (static storage, never NULL). */
const char* qlora_status_string(int status);

/* Message of the last QLORA_EHIP on the calling thread ("" if none). */
const char* qlora_last_error(void);

/* Library version string, e.g. "qlora-mi355x 0.1 gfx950". */
const char* qlora_version(void);

/* The 16 NF4 levels compiled into the library, ascending (host buffer). */
void qlora_nf4_levels(float out_host[16]);

/* K splits the library uses for a base GEMM with a plain-store epilogue
 * (output [m][n], depth k) when the base weight is bf16 in memory (the staged
 * and 16-bit paths): outputs with fewer than 256 tiles of 256 x 256 run as up
 * to 8 K ranges of at least 512, each writing fp32 partials to the workspace,
 * then one pass sums them in a fixed order and stores bf16. 1 means no split;
 * -1 for negative sizes. A pure function of the shape (workspace queries
 * include the partials), so results are deterministic. Host only. */
int qlora_gemm_split_count(int64_t m, int64_t n, int64_t k);

/* Standalone dequantization: out [n][k] bf16 = dequant(W). Bit-exact
 * contract: bf16_rne(fp32_rne(level[code] * absmax)), with the reconstructed
 * absmax for a double-quantized weight. */
int qlora_nf4_dequant(qlora_nf4 w, uint16_t* out, void* stream);

/* Double quantization of the absmax constants (the second level of the QLoRA
 * paper's storage, which the pages link): nb fp32 values (the [n][k/64] array,
 * flattened) in groups of 256 consecutive values, the last group possibly
 * shorter. Per group: offset = fp32(sum / count), the sum taken in fp64 in
 * index order; scale = fp32(max |a - offset| / 127) in fp64; each value's code
 * q = clamp(rne((a - offset) / scale), -127, 127) in fp64 (0 when scale is 0).
 * Outputs q int8 [nb], scale and offset fp32 [ceil(nb / 256)], all device
 * buffers owned by the caller; 1 byte per 64 weights plus 8 bytes per 16384.
 * Errors: QLORA_EINVAL for a NULL pointer with nb > 0, QLORA_ESHAPE for
 * nb < 0 or fp32 pointers off 4 bytes; nb == 0 does nothing. */
int qlora_absmax_dq_quantize(const float* absmax, int64_t nb, int8_t* q, float* scale,
                             float* offset, void* stream);

/* The reconstructed constants: out[i] = fp32(fp32(q[i] * scale[i/256]) +
 * offset[i/256]) (two roundings, no fused multiply-add), i < nb. Errors as
 * for qlora_absmax_dq_quantize. */
int qlora_absmax_dq_dequant(const int8_t* q, const float* scale, const float* offset, int64_t nb,
                            float* out, void* stream);

/* Quantizer: bf16 W [n][k] (k a multiple of 64, finite values) -> NF4 codes
 * [n][k/2] and absmax [n][k/64], the inverse direction of the dequant above
 * (needed to turn 16-bit weights into the 4-bit base of the method). Per
 * 64-block: absmax = max |w| (exact); each weight takes the nearest level to
 * x = w / absmax, x and the distances formed in fp64, ties to the lower
 * code; an all-zero block gets absmax 0 and code 7 (the level 0) throughout.
 * The absmax values are fp32 (qlora_absmax_dq_quantize adds the second
 * level). Layout and
 * ownership as for qlora_nf4_dequant (device pointers owned by the caller).
 * Errors: QLORA_ESHAPE if k % 64 != 0 or a size is negative or >= 2^31;
 * n*k == 0 returns QLORA_OK and touches nothing (pointers may be NULL);
 * otherwise QLORA_EINVAL for a NULL pointer, QLORA_ESHAPE unless w is
 * 16-byte and codes, absmax 4-byte aligned. Asynchronous on `stream`. */
int qlora_nf4_quantize(const uint16_t* w, int64_t n, int64_t k, uint8_t* codes, float* absmax,
                       void* stream);

/* ---------------------------------------------------------- linear layer --
 * Forward:  U = X A^T (saved, fp32 [m][r]);  Y = X W^T + s U B^T.
 * Backward: T = dY B;  dX = dY W + s T A;  dA = s T^T X;  dB = s dY^T U.
 * X [m][k], W NF4 [n][k], A [r][k], B [n][r], Y/dY [m][n], dX [m][k],
 * dA [r][k], dB [n][r]. dX may be NULL (not wanted, e.g. first layer).
 * (Mistral benchmark page, items 10-11; Reddit talk summary, "fused LoRA".) */
size_t qlora_linear_workspace_bytes(int64_t m, int64_t k, int64_t n, int64_t r, int mode);

int qlora_linear_fwd(const uint16_t* X, int64_t m, qlora_nf4 w,
                     const uint16_t* A, const uint16_t* B, int64_t r, float s,
                     uint16_t* Y, float* U_save, int mode,
                     void* ws, size_t ws_bytes, void* stream);

/* No-allocation variant of qlora_linear_fwd, for callers that cannot
 * allocate: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. Same computation, arguments, layouts, modes and errors as
 * qlora_linear_fwd, without ws / ws_bytes. Its scratch is a device array
 * inside the library, qlora_linear_fwd_noalloc_max_bytes() bytes (64 MiB) on
 * every GPU the library runs on, held from the library's load until the
 * process ends. A call whose forward needs more scratch than that (the
 * forward's share of qlora_linear_workspace_bytes(): in staged mode mostly
 * the bf16 weight copy, n * k * 2 bytes, plus fp32 K-split partials when the
 * output has fewer than 256 tiles of 256 x 256) returns QLORA_EWORKSPACE
 * before anything is enqueued, and qlora_last_error gives both sizes. The
 * 8192-token Llama-7B q_proj fits in both modes (41 MiB staged). All
 * calls on one GPU share its array and leave their contents in it: calls
 * that overlap in time on one GPU (two streams, two threads) race, and the
 * caller must order them. Nothing in the array needs to start at zero. The
 * call allocates nothing (no hipMalloc / hipFree, no stream or event); its
 * first call on a device looks up that device's copy of the array. */
size_t qlora_linear_fwd_noalloc_max_bytes(void);

int qlora_linear_fwd_noalloc(const uint16_t* X, int64_t m, qlora_nf4 w,
                             const uint16_t* A, const uint16_t* B, int64_t r, float s,
                             uint16_t* Y, float* U_save, int mode, void* stream);

int qlora_linear_bwd(const uint16_t* dY, const uint16_t* X, const float* U,
                     int64_t m, qlora_nf4 w,
                     const uint16_t* A, const uint16_t* B, int64_t r, float s,
                     uint16_t* dX, uint16_t* dA, uint16_t* dB, int mode,
                     void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------ gated MLP --
 * Forward:  g = X Wg^T + s (X Ag^T) Bg^T;  u likewise;  H = act(g) * u;
 *           Y = H Wd^T + s (H Ad^T) Bd^T.
 * Saved for the backward (caller-owned): g, u bf16 [m][h]; Ug, Uu fp32
 * [m][r] (= X Ag^T, X Au^T); Ud fp32 [m][r] (= H Ad^T). H is not saved.
 * Backward: recomputes H = act(g) * u; dH = dY Wd + s (dY Bd) Ad;
 *           dg = dH * u * act'(g); du = dH * act(g);
 *           dX = dg Wg + du Wu + s (dg Bg) Ag + s (du Bu) Au;
 *           LoRA gradients as for the linear layer, per projection.
 * (Mistral benchmark page, breakdown row "Manual Autograd MLP"; Gemma page,
 * "GeGLU vs SwiGLU activation"; Reddit talk summary, "SwiGLU" kernel.) */
size_t qlora_mlp_workspace_bytes(int64_t m, int64_t d, int64_t h, int64_t r, int mode);

int qlora_mlp_fwd(const uint16_t* X, int64_t m, const qlora_mlp_weights* w,
                  uint16_t* Y, uint16_t* g_save, uint16_t* u_save,
                  float* Ug, float* Uu, float* Ud, int mode,
                  void* ws, size_t ws_bytes, void* stream);

int qlora_mlp_bwd(const uint16_t* dY, const uint16_t* X,
                  const uint16_t* g_save, const uint16_t* u_save,
                  const float* Ug, const float* Uu, const float* Ud,
                  int64_t m, const qlora_mlp_weights* w,
                  uint16_t* dX, const qlora_mlp_grads* grads, int mode,
                  void* ws, size_t ws_bytes, void* stream);

/* --------------------------------------------------- 16-bit base weights --
 * The same linear layer and gated MLP with an unquantized bf16 base weight
 * (plain LoRA on a 16-bit model, which the pages offer beside QLoRA: Show HN
 * thread, "QLoRA / LoRA" feature list; "Introducing Unsloth", supported
 * fine-tuning modes). W [n][k] bf16 replaces the NF4 weight; everything else,
 * including the saved set, the workspace rules and the results' definition,
 * is as above. RSLoRA is the caller's choice of s (alpha / sqrt(r)).
 * The forward reads W as it is (the MLP copies gate/up into an interleaved
 * layout in the workspace); the backward transposes W into the workspace for
 * the dX product. */
size_t qlora_linear16_workspace_bytes(int64_t m, int64_t k, int64_t n, int64_t r);

int qlora_linear16_fwd(const uint16_t* X, int64_t m, const uint16_t* W, int64_t n, int64_t k,
                       const uint16_t* A, const uint16_t* B, int64_t r, float s,
                       uint16_t* Y, float* U_save, void* ws, size_t ws_bytes, void* stream);

int qlora_linear16_bwd(const uint16_t* dY, const uint16_t* X, const float* U, int64_t m,
                       const uint16_t* W, int64_t n, int64_t k,
                       const uint16_t* A, const uint16_t* B, int64_t r, float s,
                       uint16_t* dX, uint16_t* dA, uint16_t* dB,
                       void* ws, size_t ws_bytes, void* stream);

/* MLP with bf16 base weights: gate, up [h][d], down [d][h]. Passed by HOST
 * pointer. */
typedef struct qlora_mlp16_weights {
  const uint16_t* gate;
  const uint16_t* up;
  const uint16_t* down;
  const uint16_t* a_gate; /* [r][d] */
  const uint16_t* b_gate; /* [h][r] */
  const uint16_t* a_up;   /* [r][d] */
  const uint16_t* b_up;   /* [h][r] */
  const uint16_t* a_down; /* [r][h] */
  const uint16_t* b_down; /* [d][r] */
  int64_t d, h, r;
  float s;
  int act;   /* qlora_act */
} qlora_mlp16_weights;

size_t qlora_mlp16_workspace_bytes(int64_t m, int64_t d, int64_t h, int64_t r);

int qlora_mlp16_fwd(const uint16_t* X, int64_t m, const qlora_mlp16_weights* w,
                    uint16_t* Y, uint16_t* g_save, uint16_t* u_save,
                    float* Ug, float* Uu, float* Ud,
                    void* ws, size_t ws_bytes, void* stream);

int qlora_mlp16_bwd(const uint16_t* dY, const uint16_t* X,
                    const uint16_t* g_save, const uint16_t* u_save,
                    const float* Ug, const float* Uu, const float* Ud,
                    int64_t m, const qlora_mlp16_weights* w,
                    uint16_t* dX, const qlora_mlp_grads* grads,
                    void* ws, size_t ws_bytes, void* stream);

/* -------------------------------------------- q, k, v on one shared input --
 * The attention projections of a layer as one call: for p in {q, k, v},
 *   Y_p = X W_p^T + s (X A_p^T) B_p^T,   W_p [n_p][d], A_p [r][d], B_p [n_p][r],
 * X [m][d] shared (with grouped-query attention n_k, n_v < n_q). Forward: one
 * GEMM over the concatenated width n_q + n_k + n_v and one read of X for the
 * three rank-r products; saved for the backward: U fp32 [m][3r] =
 * [X A_q^T | X A_k^T | X A_v^T] (caller-owned).
 * Backward: T_p = dY_p B_p; dX = sum_p (dY_p W_p + s T_p A_p), formed as ONE
 * GEMM whose contraction runs over the three dY_p in place; dA_p = s T_p^T X;
 * dB_p = s dY_p^T U_p. dX may be NULL (not wanted).
 * (Mistral benchmark page, breakdown row "Manual Autograd QKV"; Show HN
 * thread, the author's list of savings, manual QKV autograd.)
 *   - Q, K, V (forward outputs) and dQ, dK, dV (backward inputs) each take a
 *     row pitch in elements: pitch >= n_p, a multiple of 8, pointer 16-byte
 *     aligned. They may be separate tensors or column slices of one
 *     [m][n_q + n_k + n_v] buffer; outputs must not overlap.
 *   - d, n_q, n_k, n_v: positive multiples of 64; 1 <= r <= 64.
 *   - The base weights are always dequantized (or copied, 16-bit variant)
 *     into the workspace as one bf16 [n_q + n_k + n_v][d] matrix (forward) or
 *     its transpose (backward); one workspace query serves both formats.
 *   - Errors: QLORA_EINVAL (null pointer, r, s), QLORA_ESHAPE (dimensions,
 *     mismatched d, pitch or alignment of a per-token tensor),
 *     QLORA_EWORKSPACE, QLORA_EHIP. m == 0 writes only the six LoRA
 *     gradients, as zeros; per-token pointers may then be NULL. */
typedef struct qlora_qkv_weights {
  qlora_nf4 q, k, v;      /* [n_q][d], [n_k][d], [n_v][d] */
  const uint16_t* a_q;    /* [r][d] */
  const uint16_t* b_q;    /* [n_q][r] */
  const uint16_t* a_k;    /* [r][d] */
  const uint16_t* b_k;    /* [n_k][r] */
  const uint16_t* a_v;    /* [r][d] */
  const uint16_t* b_v;    /* [n_v][r] */
  int64_t r;
  float s;
} qlora_qkv_weights;

/* The same with bf16 base weights (16-bit LoRA). */
typedef struct qlora_qkv16_weights {
  const uint16_t* q;      /* [n_q][d] */
  const uint16_t* k;      /* [n_k][d] */
  const uint16_t* v;      /* [n_v][d] */
  int64_t d, n_q, n_k, n_v;
  const uint16_t* a_q;
  const uint16_t* b_q;
  const uint16_t* a_k;
  const uint16_t* b_k;
  const uint16_t* a_v;
  const uint16_t* b_v;
  int64_t r;
  float s;
} qlora_qkv16_weights;

/* LoRA weight gradients (device pointers, bf16, shapes of the factors). */
typedef struct qlora_qkv_grads {
  uint16_t* a_q;
  uint16_t* b_q;
  uint16_t* a_k;
  uint16_t* b_k;
  uint16_t* a_v;
  uint16_t* b_v;
} qlora_qkv_grads;

size_t qlora_qkv_workspace_bytes(int64_t m, int64_t d, int64_t n_q, int64_t n_k, int64_t n_v,
                                 int64_t r);

int qlora_qkv_fwd(const uint16_t* X, int64_t m, const qlora_qkv_weights* w,
                  uint16_t* Q, int64_t ld_q, uint16_t* K, int64_t ld_k, uint16_t* V, int64_t ld_v,
                  float* U_save, void* ws, size_t ws_bytes, void* stream);

int qlora_qkv_bwd(const uint16_t* dQ, int64_t ld_dq, const uint16_t* dK, int64_t ld_dk,
                  const uint16_t* dV, int64_t ld_dv, const uint16_t* X, const float* U,
                  int64_t m, const qlora_qkv_weights* w, uint16_t* dX,
                  const qlora_qkv_grads* grads, void* ws, size_t ws_bytes, void* stream);

int qlora_qkv16_fwd(const uint16_t* X, int64_t m, const qlora_qkv16_weights* w,
                    uint16_t* Q, int64_t ld_q, uint16_t* K, int64_t ld_k, uint16_t* V,
                    int64_t ld_v, float* U_save, void* ws, size_t ws_bytes, void* stream);

int qlora_qkv16_bwd(const uint16_t* dQ, int64_t ld_dq, const uint16_t* dK, int64_t ld_dk,
                    const uint16_t* dV, int64_t ld_dv, const uint16_t* X, const float* U,
                    int64_t m, const qlora_qkv16_weights* w, uint16_t* dX,
                    const qlora_qkv_grads* grads, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------ RMS layernorm, RoPE, cross entropy --
 * The pages' other hand-derived training kernels (Mistral benchmark page,
 * breakdown items 7 "Fast RoPE Embeddings", 8 "Fast RMS Layernorm", 9 "Fast
 * Cross Entropy Loss"; Gemma page, "+1 to RMS LayerNorm" and "256K
 * vocabulary"; Reddit talk summary, "chunked cross entropy"). None of them
 * needs a workspace; every call is asynchronous on `stream`.
 *
 * RMS layernorm over rows of X [m][d] (d a multiple of 8):
 *   r_i = 1 / sqrt(mean_j x_ij^2 + eps);  Y = X * r * w'  with w' = w
 *   (gemma = 0: Llama, Mistral) or 1 + w (gemma = 1: Gemma); w [d] bf16.
 *   rstd [m] fp32 receives r for the backward (caller-owned).
 * Backward for a frozen w (LoRA trains the adapters only), g = dY * w':
 *   dX = r * (g - X * r^2 * mean_j(g_j x_j)). No gradient of w. */
int qlora_rmsnorm_fwd(const uint16_t* X, int64_t m, int64_t d, const uint16_t* w, float eps,
                      int gemma, uint16_t* Y, float* rstd, void* stream);
int qlora_rmsnorm_bwd(const uint16_t* dY, const uint16_t* X, const float* rstd, int64_t m,
                      int64_t d, const uint16_t* w, int gemma, uint16_t* dX, void* stream);

/* RoPE on X [m][heads][head_dim] (row pitch ld in elements, a multiple of 8):
 * each head vector is split into halves (a, b); with
 * theta_j = pos[i] * base^(-2j/head_dim), j < head_dim/2,
 *   Y = (a cos theta - b sin theta, b cos theta + a sin theta).
 * The backward is the transposed rotation (the angle's sign reversed):
 *   dX = (da cos + db sin, db cos - da sin).
 * pos [m] int64 (the token's position in its sequence). Angles are formed in
 * fp64 and reduced to [-pi, pi] before an fp32 sine and cosine (positions
 * never pass through bf16). head_dim a multiple of 16, at most 256. Y may be
 * X (in place, same pitch); Q and K of a fused q/k/v output can be passed
 * as column slices with its pitch. */
int qlora_rope_fwd(const uint16_t* X, int64_t ld_x, int64_t m, int64_t heads, int64_t head_dim,
                   const int64_t* pos, float base, uint16_t* Y, int64_t ld_y, void* stream);
int qlora_rope_bwd(const uint16_t* dY, int64_t ld_dy, int64_t m, int64_t heads, int64_t head_dim,
                   const int64_t* pos, float base, uint16_t* dX, int64_t ld_dx, void* stream);

/* Cross entropy of logits [m][V] bf16 (row pitch ld, a multiple of 8, >= V;
 * any V) against labels [m] int64, where a label outside [0, V) (e.g. -100)
 * marks a row without a target:
 *   lse_i = logsumexp(x_i);  ce_i = lse_i - x_i[label_i] (0 without a target);
 *   loss = sum_i ce_i / n,  n = number of rows with a target (loss 0 if n = 0).
 * Outputs: lse, ce_rows [m] fp32; loss (fp32) and n_valid (int32) are device
 * scalars, written with a fixed summation order.
 * Backward: dlogits = (softmax(x_i) - onehot(label_i)) * dloss / n for rows
 * with a target, 0 otherwise; dloss is a device fp32 scalar (NULL = 1.0);
 * n_valid and lse as written by the forward. dlogits may be logits (in place,
 * same pitch). Errors: QLORA_ESHAPE for sizes, pitches or alignment (bf16
 * arrays 16-byte aligned), QLORA_EINVAL for NULL pointers. */
int qlora_cross_entropy_fwd(const uint16_t* logits, int64_t ld, int64_t m, int64_t V,
                            const int64_t* labels, float* lse, float* ce_rows, float* loss,
                            int32_t* n_valid, void* stream);
int qlora_cross_entropy_bwd(const uint16_t* logits, int64_t ld, int64_t m, int64_t V,
                            const int64_t* labels, const float* lse, const float* dloss,
                            const int32_t* n_valid, uint16_t* dlogits, int64_t ld_d, void* stream);

/* Forward and backward in one call, for when the upstream gradient of the
 * loss is known before the loss itself (training: 1, or a loss scale): the
 * outputs of qlora_cross_entropy_fwd plus dlogits for dloss given as a host
 * float, with the same bits as the two separate calls. Each row of logits is
 * read from HBM once (the gradient pass re-reads it from cache), 2 B per
 * logit instead of 4 over the pair. dlogits may be logits (in place, same
 * pitch). Errors as for the separate calls; dloss must be finite. */
int qlora_cross_entropy_fused(const uint16_t* logits, int64_t ld, int64_t m, int64_t V,
                              const int64_t* labels, float dloss, float* lse, float* ce_rows,
                              float* loss, int32_t* n_valid, uint16_t* dlogits, int64_t ld_d,
                              void* stream);

/* ---------------------------------------------------------------- tracing --
 * Kernel timing aid for benchmarks and profiling. While enabled, every
 * dense-contraction (base GEMM) launch made by the entry points above is
 * bracketed by a pair of HIP events recorded on the launch stream, together
 * with its algorithmic FLOP count (2 m n k of the base product plus
 * 2 m n r of the LoRA term it carries). Enabling/disabling and reading are
 * host calls; reading waits for the recorded events. Not thread-safe with
 * concurrent entry-point calls. Disabled by default; costs nothing when off.
 *   qlora_trace_enable(1) clears previous records and starts recording.
 *   qlora_trace_read(...) returns the number of recorded launches, their
 *   summed GPU time in milliseconds and summed algorithmic FLOPs. */
int qlora_trace_enable(int on);
int qlora_trace_read(int64_t* launches, double* total_ms, double* total_flops);

/* ------------------------------------------------------------ diagnostics --
 * Measures the sustained dense bf16 matrix-core rate of the current device:
 * 8 blocks of 4 waves per CU, each wave running 8 independent chains of
 * 32x32x16 bf16 MFMAs, `iters` rounds, on operands with random bits. Reports
 * the best of three timed launches (after one warm-up) in TFLOP/s and the
 * shader clock in GHz read on one wave under that load. Enqueues on `stream`
 * and waits for it (blocking host call). Allocates nothing.
 * Errors: QLORA_EINVAL (null outputs, iters < 1), QLORA_EHIP. */
int qlora_probe_mfma_peak(int iters, double* tflops, double* shader_ghz, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_H */
