/*
 * moe_decode.h - C ABI of the MI355X (gfx950) quantized MoE decode library.
 *
 * What it computes (one MoE FFN layer, per token row t, rows independent):
 *   u_t      = h_t / sqrt(mean(h_t^2) + eps)                 RMS normalisation, weight 1
 *   logits   = W_r u_t                                       router GEMV
 *   ids, w   = top-k of logits (descending, ties -> lower id);
 *              w = softmax restricted to the k selected logits (renormalised)
 *   a_e      = silu(W_gate,e u_t) * (W_up,e u_t)             SwiGLU, each selected expert e
 *   a_s      = the same for the shared expert
 *   out_t    = h_t + sum_i w_i W_down,ids_i a_ids_i + sigmoid(gvec . u_t) W_down,s a_s
 *   h_out_t  = bf16(out_t), round to nearest even
 * Sources: PureDrive-35B-A3B-MLX model card, "Summary" (top-8 of 256 routed
 * experts plus one shared expert; 6-bit routed, 8-bit shared/router) and "FAQ"
 * (every selected expert runs); flash-moe news page (ja.news.hada.io topic
 * 27758), "FMA-optimised dequant kernel" (weight = code*scale + bias, group
 * affine), "Metal Compute Shaders" (SwiGLU, RMS normalisation, MoE combine +
 * residual + gate) and "Deferred GPU Expert Compute" (combine, norm and
 * residual stay on the GPU and feed the next layer directly).
 *
 * Conventions for every entry point:
 *   - return 0 (MOE_OK) on success or a negative MOE_ERR_* code; the message
 *     of the last failure on the calling thread is moe_last_error().
 *   - all argument validation is host code and runs before any launch; a
 *     failed validation launches nothing and touches no buffer.
 *   - "dev" pointers are device (HBM) addresses, "host" pointers host
 *     addresses. The caller owns every buffer; the library never allocates
 *     device memory. It keeps no pointer beyond a call, except that
 *     moe_stack_init writes a descriptor table of layer pointers into the
 *     caller's workspace and fills a caller-owned moe_stack_t.
 *   - launches are asynchronous on the given stream (a hipStream_t, NULL =
 *     the default stream); device-side faults surface at the caller's next
 *     synchronisation. With MOE_DEBUG_SYNC=1 in the environment (read once,
 *     at the first call), every entry point that launches work waits for its
 *     stream before returning and turns a HIP error into MOE_ERR_HIP, and a
 *     stack call whose bounded waits timed out returns MOE_ERR_TIMEOUT.
 *   - results are bitwise deterministic, and for T <= 8 row t of a T-row
 *     call is bitwise equal to a T = 1 call on that row alone.
 */
#ifndef MOE_DECODE_H
#define MOE_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* moe_stream_t; /* a hipStream_t */

enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1,     /* null pointer, bad size, bad shape field */
  MOE_ERR_UNSUPPORTED = -2,     /* bit width / group / dimension not supported */
  MOE_ERR_ALIGNMENT = -3,       /* device pointer not aligned as documented */
  MOE_ERR_WORKSPACE = -4,       /* workspace smaller than moe_workspace_bytes() */
  MOE_ERR_HIP = -5,             /* a HIP runtime call failed */
  MOE_ERR_TIMEOUT = -6          /* (MOE_DEBUG_SYNC only) a bounded cross-workgroup wait timed out */
};

/* Shape of one MoE layer. Limits: hidden, inter, shared_inter multiples of 64
 * in [64, 8192]; 1 <= top_k <= min(n_experts, 16); n_experts <= 512;
 * expert_bits, shared_bits in {2, 3, 4, 6, 8}; router_bits in {2, 3, 4, 6, 8}
 * or 16 (dense bf16 router); group must be 64; rms_eps > 0.
 * The fields follow the PureDrive card, "Summary" (256 experts, top-8 plus a
 * shared expert, 6-bit experts and 8-bit shared expert/router) and the
 * flash-moe news page, "Model architecture" (512 experts, hidden 4096) and
 * "FMA-optimised dequant kernel" (group-affine 4-bit and 2-bit weights). */
typedef struct moe_shape {
  int32_t hidden;        /* H */
  int32_t n_experts;     /* E routed experts */
  int32_t inter;         /* I, routed expert intermediate size */
  int32_t top_k;         /* k */
  int32_t shared_inter;  /* I_s, shared expert intermediate size */
  int32_t router_bits;   /* 16 = dense bf16 [E, H]; else group-affine codes */
  int32_t expert_bits;
  int32_t shared_bits;
  int32_t group;         /* 64 */
  float rms_eps;         /* 1e-6 */
} moe_shape_t;

/*
 * Packed quantised matrix W [rows, cols], group-affine along cols in groups of
 * 64: W[r, c] = code[r, c] * scale[r, c/64] + bias[r, c/64] (flash-moe news
 * page, "FMA-optimised dequant kernel"). One matrix block is
 *   codes  : rows * row_bytes(bits, cols), row-major, rows back to back
 *   (pad)  : to a multiple of 256 bytes
 *   sb     : rows * (cols/64) dwords; dword = scale bf16 (bits 0-15) |
 *            bias bf16 (bits 16-31), row-major
 *   (pad)  : to a multiple of 256 bytes
 * Codes inside a row (code j = column j):
 *   bits 2, 4, 8 : dense, LSB first: code j at bit offset bits*j of the row.
 *   bits 6       : units of 16 codes in 3 dwords A, B, C. Unit u holds
 *                  codes 16u..16u+15; local code c = j + 8h (h in {0,1},
 *                  j in 0..7) lives in bits 16h..16h+15 of the dwords, at
 *                  these offsets within that half: j = 0, 1: A bit 6j;
 *                  j = 3, 4: B bit 6(j-3); j = 6, 7: C bit 6(j-6) (all 6
 *                  bits); j = 2: low 4 bits at A bit 12, high 2 bits at C
 *                  bit 12; j = 5: low 4 bits at B bit 12, high 2 bits at C
 *                  bit 14. (Codes c and c+8 share bit positions, so one mask
 *                  extracts both halves of a decode pair.)
 *   bits 3       : 10 codes per dword, code j in dword j/10; with
 *                  l = j%10 at bit 3l for l < 5 and at bit 16 + 3(l-5) for
 *                  l >= 5 (codes l and l+5 share bit positions in the two
 *                  halves); bits 15 and 31 zero; each row padded to whole
 *                  dwords with zero.
 * row_bytes = cols*bits/8 for bits 2/4/6/8, 4*ceil(cols/10) for bits 3.
 * Returns the block's bytes, or a negative MOE_ERR_* code.
 */
int64_t moe_matrix_bytes(int32_t bits, int32_t rows, int32_t cols);

/* Byte offsets of the parts of one layer block (each 256-byte aligned):
 * router (packed matrix [E, H], or dense bf16 [E, H] when router_bits = 16),
 * gate vector (bf16 [H]), shared expert, then routed expert e at
 * expert0 + e * expert_stride. An expert is three packed matrices back to
 * back: gate [I, H], up [I, H], down [H, I]. One contiguous block per expert
 * is what the flash-moe news page, "SSD Expert Streaming", reads per selected
 * expert (about 6.75 MB at the 397B shape, 4-bit). */
typedef struct moe_layer_layout {
  int64_t router;
  int64_t gatevec;
  int64_t shared;         /* shared expert block */
  int64_t shared_up;      /* offsets of up / down inside an expert block */
  int64_t shared_down;
  int64_t expert0;
  int64_t expert_stride;
  int64_t expert_up;
  int64_t expert_down;
  int64_t total_bytes;    /* whole layer block */
} moe_layer_layout_t;

/* Validates the shape (pure host code, no device). */
int32_t moe_validate_shape(const moe_shape_t* shape);

/* Validates the shape and a row count 1 <= T <= 32 (pure host code, no
 * device). T is the number of token rows of one call: 1 for decode, up to 8
 * for the verify pass of the PureDrive card, "How it works" (3 rows there),
 * up to 32 for batches. */
int32_t moe_validate(const moe_shape_t* shape, int32_t T);

/* Fills *out (host) for a valid shape. */
int32_t moe_layer_layout(const moe_shape_t* shape, moe_layer_layout_t* out);

/* Bytes of one routed expert block (gate, up and down packed matrices with
 * their padding; the layout's expert_stride), e.g. 7,077,888 = 6.75 MiB at
 * the 397B shape with 4-bit codes (flash-moe news page, "SSD Expert
 * Streaming": about 6.75 MB per expert). Negative MOE_ERR_* on a bad shape. */
int64_t moe_expert_bytes(const moe_shape_t* shape);

/* Bytes of one whole layer block (router, gate vector, shared expert and all
 * routed experts). Negative MOE_ERR_* on a bad shape. */
int64_t moe_layer_bytes(const moe_shape_t* shape);

/* Bytes of workspace for calls of up to T rows (1 <= T <= 32) on stacks of
 * up to n_layers layers (n_layers = 0: moe_decode_layer and moe_decode_stack
 * only; n_layers >= 1 adds the descriptor table moe_stack_init writes). The
 * same workspace serves every decode entry point. Negative MOE_ERR_* on an
 * invalid shape, T or n_layers (0 <= n_layers <= 4096). */
int64_t moe_workspace_bytes(const moe_shape_t* shape, int32_t n_layers, int32_t T);

/* Host-side packing of one matrix into the layout above.
 * codes_host: uint8 [rows, cols], each < 2^bits; scale_host, bias_host: bf16
 * bit patterns [rows, cols/64]; dst_host: moe_matrix_bytes() bytes, fully
 * written (padding zero). cols must be a multiple of 64. A code >= 2^bits
 * returns MOE_ERR_INVALID_ARG with dst partly written. The group-affine form
 * is the flash-moe news page's, "FMA-optimised dequant kernel". */
int32_t moe_pack_matrix(int32_t bits, int32_t rows, int32_t cols, const uint8_t* codes_host,
                        const uint16_t* scale_host, const uint16_t* bias_host, void* dst_host);

/* Inverse of moe_pack_matrix (host only; same arguments, outputs written). */
int32_t moe_unpack_matrix(int32_t bits, int32_t rows, int32_t cols, const void* src_host,
                          uint8_t* codes_host, uint16_t* scale_host, uint16_t* bias_host);

/*
 * Synthetic weights: writes the whole layer block of layer `layer` on the
 * device (layer_dev: moe_layer_bytes() bytes, 256-byte aligned), drawing
 * codes, bf16 scales/biases and bf16 vectors from the seeded splitmix64
 * counter generator (Steele, Lea & Flood, OOPSLA 2014) with per-(layer,
 * expert) sub-seeds. The pages publish no weights (PureDrive card: the
 * repository holds documentation only); the definition of the draws is the
 * one documented with the library sources (gen kernels).
 */
int32_t moe_generate_layer(const moe_shape_t* shape, uint64_t seed, int32_t layer, void* layer_dev,
                           moe_stream_t stream);

/* Synthetic x rows: bf16 [T, H] ~ N(0, 1) from seed_x, written to out_dev
 * (16-byte aligned), as the generator above. */
int32_t moe_generate_rows(uint64_t seed_x, int32_t T, int32_t H, uint16_t* out_dev, moe_stream_t stream);

/*
 * One MoE layer on T rows (1 <= T <= 32): the whole step of the header
 * comment, i.e. the router GEMV, softmax top-k, the selected experts' and the
 * shared expert's dequantised SwiGLU GEMVs and the combine + residual + gate
 * of the flash-moe news page, "Metal Compute Shaders" and "Deferred GPU
 * Expert Compute", with only the router-selected experts read (AiiStream
 * news page: the router's choice decides which experts are loaded).
 *   layer_dev : layer block (layout above), 256-byte aligned
 *   h_in_dev  : bf16 [T, H], 16-byte aligned; h_out_dev: bf16 [T, H], 16-byte
 *               aligned, must not overlap h_in_dev
 *   ids_dev   : int32 [T, k] selected experts (descending logit) or NULL
 *   w_dev     : float [T, k] renormalised routing weights or NULL
 *   ws_dev    : workspace of ws_bytes >= moe_workspace_bytes(shape, 0, T),
 *               256-byte aligned; contents need no initialisation.
 * Calls that share one workspace must be ordered on one stream.
 * Rows are independent. For T <= 8 (the verify batch of the PureDrive card,
 * "How it works") row t of the result is bitwise equal to a one-row call on
 * row t. For T > 8 with an 8-bit router and shared expert, those two run on
 * the bf16 matrix cores (different fp32 summation order; rows agree with the
 * one-row result to rounding, not bit for bit).
 */
int32_t moe_decode_layer(const moe_shape_t* shape, const void* layer_dev, int32_t T, const uint16_t* h_in_dev,
                         uint16_t* h_out_dev, int32_t* ids_dev, float* w_dev, void* ws_dev, size_t ws_bytes,
                         moe_stream_t stream);

/*
 * A stack of n_layers MoE layers with distinct weights: h_0 = h_in,
 * h_{l+1} = bf16(layer_l(h_l)), h_out = h_{n_layers}. Each layer's combined
 * output is handed to the next layer on the GPU (flash-moe news page,
 * "Deferred GPU Expert Compute"), and no host work or per-layer submission
 * sits between layers (the per-layer command-buffer gap the M5 Max news page,
 * "Effective optimisations", removes by pre-encoding). For T = 1 each group
 * of up to 64 layers runs as one kernel with one workgroup per compute unit,
 * whose workgroups wait on each other's results (bounded waits; see
 * moe_stack_status); it is launched only when the device can hold all its
 * workgroups at once, else the call runs as kernels per layer (the same as
 * moe_decode_layer). Both give the same results bit for bit.
 *   layers_host : host array of n_layers device pointers to layer blocks
 *                 (read during the call only)
 *   ids_dev     : int32 [n_layers, T, k] or NULL; w_dev: float [n_layers, T, k] or NULL
 *   h_trace_dev : bf16 [n_layers + 1, T, H] (h_0 .. h_L) or NULL
 *   ws_dev      : ws_bytes >= moe_workspace_bytes(shape, 0, T)
 * Other arguments as for moe_decode_layer.
 */
int32_t moe_decode_stack(const moe_shape_t* shape, const void* const* layers_host, int32_t n_layers, int32_t T,
                         const uint16_t* h_in_dev, uint16_t* h_out_dev, int32_t* ids_dev, float* w_dev,
                         uint16_t* h_trace_dev, void* ws_dev, size_t ws_bytes, moe_stream_t stream);

/* Path selection of an initialised stack (moe_stack_init flags). */
enum {
  MOE_PATH_DEFAULT = 0,
  MOE_PATH_PER_LAYER = 1,  /* T = 1 calls also run as kernels per layer (no persistent kernel) */
  MOE_PATH_NO_MFMA = 2     /* batches of T > 8 keep the router and shared expert on the vector units */
};

/* State of an initialised stack: plain host data owned by the caller (may be
 * copied); filled by moe_stack_init, read by moe_stack_decode. */
typedef struct moe_stack {
  moe_shape_t shape;
  int32_t n_layers;
  int32_t t_max;
  int32_t flags;
  uint32_t magic;        /* set by moe_stack_init */
  void* ws_dev;
  size_t ws_bytes;
  int64_t table_offset;  /* bytes from ws_dev to the descriptor table */
  int64_t reserved[4];
} moe_stack_t;

/*
 * Prepares repeated decoding of one stack (the stack of moe_decode_stack,
 * with its layer list fixed once, as a command sequence encoded once is
 * replayed per token on the M5 Max news page, "Effective optimisations"):
 * validates the shape, n_layers (1..4096), t_max (1..32) and flags, writes
 * the descriptor table (the n_layers device pointers of layers_host, each
 * 256-byte aligned) into the workspace with a kernel on `stream`, and fills
 * *st. ws_bytes >= moe_workspace_bytes(shape, n_layers, t_max). Later calls
 * that use *st must be ordered after this one (same stream, or synchronised).
 * moe_decode_layer and moe_decode_stack calls on the same workspace leave the
 * table intact.
 */
int32_t moe_stack_init(moe_stack_t* st, const moe_shape_t* shape, const void* const* layers_host, int32_t n_layers,
                       int32_t t_max, int32_t flags, void* ws_dev, size_t ws_bytes, moe_stream_t stream);

/*
 * One decode step of an initialised stack on T <= st->t_max rows: the same
 * computation and results as moe_decode_stack over the stack's layers (ids,
 * w, h_trace as there, sized by st->n_layers), with the layer pointers read
 * from the descriptor table in the workspace.
 */
int32_t moe_stack_decode(const moe_stack_t* st, int32_t T, const uint16_t* h_in_dev, uint16_t* h_out_dev,
                         int32_t* ids_dev, float* w_dev, uint16_t* h_trace_dev, moe_stream_t stream);

/*
 * Reads the status word the last stack call (moe_decode_stack or
 * moe_stack_decode) on this workspace left, into *status_host (waits for the
 * stream first): 0 = every cross-workgroup wait was met; 1 = a wait timed out
 * (about a second without progress, e.g. when other work kept part of the
 * stack kernel's workgroups off the device), the call's outputs are then
 * invalid. The word is cleared once per stack call, so a time-out in any of
 * the call's launches is reported. T must be the T of that call.
 */
int32_t moe_stack_status(const moe_shape_t* shape, int32_t T, const void* ws_dev, uint32_t* status_host,
                         moe_stream_t stream);

/*
 * moe_decode_stack for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments, computation and results, but no workspace argument:
 * the workspace is a static device array inside the library, 4 MiB per GPU,
 * held from the first call on that GPU until the process ends. The call
 * allocates nothing (no hipMalloc / hipFree, no allocating library routine).
 * A shape and T whose workspace (moe_workspace_bytes(shape, 0, T)) exceeds
 * 4 MiB is rejected with MOE_ERR_WORKSPACE before anything is launched (every
 * shape of 2048 or 4096 hidden here fits at T = 32). Every call on one GPU
 * uses that GPU's one array: calls that overlap on one GPU (different
 * streams, or host threads without ordering) race and give undefined
 * results; calls ordered on one stream are safe. moe_stack_status does not
 * read this array.
 */
int32_t moe_decode_stack_static(const moe_shape_t* shape, const void* const* layers_host, int32_t n_layers,
                                int32_t T, const uint16_t* h_in_dev, uint16_t* h_out_dev, int32_t* ids_dev,
                                float* w_dev, uint16_t* h_trace_dev, moe_stream_t stream);

/*
 * Dense projections (the non-expert weights): y_m = W_m x for n_mats
 * group-affine matrices W_m [rows_m, cols] that share one input x, computed
 * in one launch that reads x once (the fused Q/K/V projection kernel of the
 * Qwen3.5-397B on M5 Max news page, "Effective optimisations"); the attention
 * output projection and lm_head are the one-matrix case (8-bit on the
 * PureDrive card, "Summary"). W_m[r, c] = code * scale + bias in groups of 64
 * along c (flash-moe news page, "FMA-optimised dequant kernel").
 *   bits      : code width of every matrix of the call, {2, 3, 4, 6, 8}
 *   cols      : K, a multiple of 64 in [64, 8192]
 *   T         : token rows, 1 <= T <= 32
 *   x_dev     : bf16 [T, cols], 16-byte aligned
 *   mats_host : host array of n_mats (1..4) descriptors: w_dev a packed
 *               matrix block (moe_matrix_bytes layout, 256-byte aligned),
 *               rows_m in [1, 2^22] (all matrices together at most 2^22),
 *               y_dev fp32 [T, rows_m] (4-byte aligned, overlapping neither
 *               x nor another output)
 * Results are fp32 and not rounded; row t of a T-row call equals a one-row
 * call on row t bit for bit.
 */
typedef struct moe_gemv_mat {
  const void* w_dev;
  int32_t rows;
  int32_t reserved;
  float* y_dev;
} moe_gemv_mat_t;

int32_t moe_gemv(int32_t bits, int32_t cols, int32_t T, const uint16_t* x_dev, const moe_gemv_mat_t* mats_host,
                 int32_t n_mats, moe_stream_t stream);

/*
 * Synthetic dense projection: writes one packed matrix [rows, cols] with
 * `bits`-bit codes (moe_matrix_bytes bytes at dst_dev, 256-byte aligned) from
 * the generator of moe_generate_layer, with the sub-seed of (seed, layer,
 * slot 2^20 - 1) and the draw stream of `tensor` (query 6, key 7, value 8,
 * attention output 9, lm_head 10; any id in [6, 1023] is accepted).
 */
int32_t moe_generate_matrix(int32_t bits, int32_t rows, int32_t cols, uint64_t seed, int32_t layer, int32_t tensor,
                            void* dst_dev, moe_stream_t stream);

/*
 * Grouped-query decode attention of T verify rows over a bf16 K/V cache
 * (PureDrive card, "How it works": K/V read once for all query heads of a KV
 * head and all verify rows, split along the keys with split points and
 * summation order that depend only on the row's position; "Beyond this
 * checkpoint": 16 query heads, 2 KV heads, head dimension 256). Row i is at
 * position p0 + i and attends to positions 0 .. p0 + i:
 *   o[i, h] = sum_j softmax_j(q[i, h] . K[h / g, j] / sqrt(d)) V[h / g, j],
 * g = n_q / n_kv. The keys are split at fixed multiples of a chunk that
 * depends on the cache alone (head_dim 64 and 128: 512 positions; head_dim
 * 256: the largest of 512, 256, 128 and 64 positions that gives at least 512
 * chunks x KV heads over max_seq, else 64), so row i of a T-row call equals a
 * one-row call with p0 + i on the same cache bit for bit. At
 * head_dim 256 each chunk's K and V are read once for all T x g queries of a
 * KV head (the scores and the weighted values on the matrix cores, the
 * probabilities entering the latter as two bf16 parts, exact to 2^-18
 * relative); at head_dim 64 and 128 once per pass of up to 16 queries (whole
 * verify rows).
 *   shape  : n_q, n_kv with n_q a multiple of n_kv, n_q / n_kv <= 16 (<= 8
 *            at head_dim 256), n_q <= 128; head_dim in {64, 128, 256};
 *            max_seq (cache length)
 *            in [1, 2^24]
 *   T      : 1..8 rows; p0 >= 0 with p0 + T <= max_seq
 *   q_dev  : bf16 [T, n_q, head_dim]; k_dev, v_dev: bf16 [n_kv, max_seq,
 *            head_dim] (positions 0 .. p0 + T - 1 filled with finite values;
 *            the rest is not read); o_dev: fp32 [T, n_q, head_dim]; all
 *            16-byte aligned
 *   ws_dev : ws_bytes >= moe_gqa_workspace_bytes(shape, T), 256-byte aligned
 */
typedef struct moe_attn_shape {
  int32_t n_q;
  int32_t n_kv;
  int32_t head_dim;
  int32_t max_seq;
} moe_attn_shape_t;

int64_t moe_gqa_workspace_bytes(const moe_attn_shape_t* shape, int32_t T);

int32_t moe_gqa_decode(const moe_attn_shape_t* shape, int32_t T, int32_t p0, const uint16_t* q_dev,
                       const uint16_t* k_dev, const uint16_t* v_dev, float* o_dev, void* ws_dev, size_t ws_bytes,
                       moe_stream_t stream);

/*
 * One decode step of the Gated DeltaNet layers' recurrence for T tokens in
 * order (PureDrive card, "Summary": 30 Gated DeltaNet layers in the 35B-A3B
 * model; flash-moe news page, "Accelerate BLAS活用": the recurrence as
 * cblas_sscal / cblas_sgemv / cblas_sger), the gated delta rule of Yang,
 * Kautz & Hatamizadeh (ICLR 2025): for each value head h with key head
 * kh = h / (n_v / n_k) and each token t,
 *   S_h <- alpha[t,h] S_h;  u = S_h k[t,kh];
 *   S_h <- S_h + beta[t,h] (v[t,h] - u) k[t,kh]^T;  o[t,h] = S_h q[t,kh].
 * q and k arrive normalised (the projections, convolution and normalisation
 * before the recurrence are not part of this step). Token t of a T-token call
 * equals the t-th of T one-token calls in order, bit for bit.
 *   shape     : d_k in {64, 128, 256}; d_v in [1, 4096]; n_v a multiple of
 *               n_k, n_v <= 1024
 *   state_dev : fp32 [n_v, d_v, d_k], read and overwritten with the state
 *               after the last token (16-byte aligned)
 *   q_dev, k_dev : fp32 [T, n_k, d_k] (16-byte aligned); v_dev: fp32
 *               [T, n_v, d_v]; alpha_dev, beta_dev: fp32 [T, n_v]; o_dev:
 *               fp32 [T, n_v, d_v]; the inputs must not overlap the state or
 *               o; 1 <= T <= 32
 */
typedef struct moe_gdn_shape {
  int32_t n_k;
  int32_t n_v;
  int32_t d_k;
  int32_t d_v;
} moe_gdn_shape_t;

int32_t moe_gdn_step(const moe_gdn_shape_t* shape, int32_t T, float* state_dev, const float* q_dev,
                     const float* k_dev, const float* v_dev, const float* alpha_dev, const float* beta_dev,
                     float* o_dev, moe_stream_t stream);

/* Message for the last failure on this thread ("" if none). Valid until the
 * thread's next call into the library. */
const char* moe_last_error(void);

/* Library version string; ends in " debug-sync" when MOE_DEBUG_SYNC=1 was
 * seen at the first call. */
const char* moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_DECODE_H */
