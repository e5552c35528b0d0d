/*
 * moe.h — C ABI of the MI355X (gfx950) mixture-of-experts layer library, libmoe.so.
 *
 * The layer is the MoE block of the ZONOS2 and ZONOS3-Mini TTS backbones:
 *   router logits -> top-k expert selection + routing weights -> dispatch (grouping of the
 *   token-to-expert assignments by expert) -> per-expert SwiGLU FFN -> weighted combine.
 *
 * Sources of the definitions (cited by page title and section):
 *   - zonos2.cpp INTERNALS, "Model architecture" table, MoE row: 16 experts, top-1.
 *   - zonos2.cpp INTERNALS, "Model architecture" table, Router row: prob-weighted, no-renorm
 *     top-k (ZONOS2 scoring: softmax over all experts, each chosen expert weighted by its full
 *     probability).
 *   - audio.cpp PR #1271 "New Community Model: ZONOS3-Mini", "Framework change": SelectedSoftmax
 *     scoring (rank experts by raw logit plus a per-expert selection bias, take the top k, then
 *     weight them by the softmax of their raw logits over the selected set only).
 *   - audio.cpp PR #1271, "Summary": top-2-of-64 MoE at width 1024; SwiGLU FFN.
 *   - zonos2.cpp INTERNALS, "Recommended: F16 spine + K-quant experts": expert weights are
 *     3-D gate/up/down stacks.
 *   - zonos2.cpp INTERNALS, "Notes": activation and residual streams are F32; token-major
 *     [T, C] activations (ggml's [C, T] in reversed order).
 *   - zonos2.cpp INTERNALS, "Performance": the decode graph is replayed as a captured graph,
 *     so every call here is capturable (no host synchronisation, no allocation).
 *
 * Conventions shared by every entry point
 *   Pointers     Every tensor pointer is a DEVICE pointer, borrowed for the duration of the
 *                stream work the call enqueues. The library allocates nothing and keeps no
 *                state between calls; buffers must stay alive until the stream has passed the
 *                call. Tensors are dense row-major (C order) with no padding.
 *   Alignment    Every tensor pointer must be 16-byte aligned (MOE_ERR_SHAPE otherwise).
 *   Stream       `stream` is a hipStream_t passed as void* (NULL = the null stream). Every call is
 *                asynchronous: it only enqueues kernels. No call reads device memory on the host,
 *                synchronises, or allocates, so every call may be captured into a HIP graph.
 *                Launch shapes depend only on the scalar arguments, never on routing results.
 *   Dtypes       `dtype` (MOE_F32 or MOE_BF16) is the type of x and of every weight matrix
 *                (the layer's expert stacks may instead be in a prepared decode format:
 *                moe_layer_args.w_dtype, moe_quantize_*, moe_pack_weights_frag). Logits, biases, routing weights and expert outputs are always fp32; y is fp32
 *                unless a `y_dtype` argument asks for bf16 (the sum is formed in fp32 and
 *                rounded once to nearest even).
 *   Errors       A negative return means nothing was enqueued, except MOE_ERR_HIP, which reports
 *                a failed launch (work enqueued before it by the same call may have run).
 *                Device data is never validated: NaN logits or expert ids outside [0, E) are
 *                outside the contract. No C++ exception crosses this interface.
 *   Shapes       1 <= E <= 256, 1 <= k <= min(E, 8), 0 <= T <= 2^24 (T == 0 enqueues nothing
 *                and returns MOE_OK), d and H multiples of 64 (bf16) or of 4 (fp32) and at most
 *                65536, and T * k * max(d, H) < 2^31 (every activation-sized buffer has fewer
 *                than 2^31 elements; this keeps every launch within the hardware's grid limits).
 *                Violations return MOE_ERR_SHAPE / MOE_ERR_UNSUPPORTED.
 *   Reentrancy   Stateless and thread-safe; calls on different streams may run concurrently
 *                when their buffers do not overlap.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 5

enum moe_status {
  MOE_OK = 0,
  MOE_ERR_NULL = -1,        /* a required pointer is NULL                                    */
  MOE_ERR_SHAPE = -2,       /* a size is out of range, or a pointer is not 16-byte aligned   */
  MOE_ERR_UNSUPPORTED = -3, /* unknown dtype/scoring, or an argument combination not defined */
  MOE_ERR_WORKSPACE = -4,   /* workspace pointer NULL or smaller than moe_workspace_size()   */
  MOE_ERR_HIP = -5          /* a HIP launch failed                                           */
};

enum moe_dtype {
  MOE_F32 = 0,
  MOE_BF16 = 1,
  /* int8 expert weights with one fp32 scale per weight row (moe_quantize_rows_i8). Only as
     moe_layer_args.w_dtype, with bf16 activations, on the decode path. Added in ABI 2. */
  MOE_I8 = 2,
  /* 4-bit affine expert weights, one bf16 (scale, bias) pair per group of 64 along the reduction
     index, codes in the packed order of moe_quantize_groups_q4. Only as moe_layer_args.w_dtype,
     with bf16 activations, on the decode path. Added in ABI 3. */
  MOE_Q4 = 3,
  /* bf16 expert weights, int8 codes (with MOE_I8's scales) or packed 4-bit codes (with MOE_Q4's
     (scale, bias) pairs) in the fragment-major order of moe_pack_weights_frag (the same bytes,
     reordered). Only as moe_layer_args.w_dtype, with bf16 activations; MOE_BF16_FRAG on every
     shape, the codes on the decode path only. Added in ABI 5. */
  MOE_BF16_FRAG = 4,
  MOE_I8_FRAG = 5,
  MOE_Q4_FRAG = 6
};

enum moe_scoring {
  /* ZONOS2 (zonos2.cpp INTERNALS, "Model architecture", Router row): rank experts by logit
     (equivalently by softmax probability), weight each chosen expert by its softmax probability
     over ALL E experts, no renormalisation. sel_bias must be NULL in this mode. */
  MOE_SCORING_SOFTMAX = 0,
  /* ZONOS3-Mini (audio.cpp PR #1271, "Framework change"): rank by fp32(logit + sel_bias[e])
     (one round-to-nearest-even add), take the top k, weight them by the softmax of their raw
     logits over the k selected experts only (weights sum to 1; k = 1 gives exactly 1). */
  MOE_SCORING_SELECTED_SOFTMAX = 1,
  /* Sigmoid scoring, the other pre-ranking mode that audio.cpp's MoE routing already has (audio.cpp
     PR #1271, "Framework change": the existing modes apply softmax or sigmoid before ranking):
     rank by logit (the order of sigmoid(logit) in exact arithmetic; fp32 sigmoid saturates to 1
     and would create ties), weight each chosen expert by sigmoid(logit) = 1 / (1 + exp(-logit)),
     no renormalisation (the weights need not sum to 1). sel_bias must be NULL. Added in ABI 2. */
  MOE_SCORING_SIGMOID = 2
};

/* Returns MOE_ABI_VERSION of the built library. */
int moe_abi_version(void);

/* Static text for a status code (never NULL). */
const char* moe_status_string(int status);

/* Bytes of device workspace that moe_expert_ffn and moe_layer_forward need for these sizes
   (0 when T == 0). The value depends only on the arguments. Returns 0 for invalid sizes. */
size_t moe_workspace_size(int T, int d, int E, int H, int k, int dtype);

/*
 * Router logits, step 1 (zonos2.cpp INTERNALS, "Model architecture", Router row; the router here
 * is a plain linear map, the pages do not define the EDA router's internals):
 *   logits[t, e] = sum_i x[t, i] * w_router[e, i] + router_bias[e]
 *   x         [T, d]  dtype      token activations
 *   w_router  [E, d]  dtype      router weight
 *   router_bias [E]   fp32/NULL  added to every token's logits (NULL = no bias)
 *   logits    [T, E]  fp32       output; accumulated in fp32 (bf16 products are exact in fp32)
 * Sizes: 0 <= T <= 2^24, 1 <= E <= 256, d a multiple of 64 (bf16) or 4 (fp32), T * d < 2^31.
 */
int moe_router_logits(const void* x, const void* w_router, const float* router_bias,
                      int T, int d, int E, int dtype, float* logits, void* stream);

/*
 * Routing, steps 2-3: top-k selection, routing weights and per-expert counts on GIVEN fp32 logits
 * (audio.cpp PR #1271, "Framework change"; zonos2.cpp INTERNALS, "Model architecture", Router
 * row). Selection orders experts by (score descending, expert index ascending), where
 * score = logits (SOFTMAX) or fp32(logits + sel_bias) (SELECTED_SOFTMAX); -0.0 equals +0.0.
 * Slot 0 holds the best expert. Indices and counts are exact integers: identical logits give
 * identical results on every call.
 *   logits        [T, E] fp32   input
 *   sel_bias      [E]    fp32   SELECTED_SOFTMAX only (may be NULL = zero bias); must be NULL
 *                               for SOFTMAX (MOE_ERR_UNSUPPORTED otherwise)
 *   topk_ids      [T, k] int32  output, expert id per slot
 *   topk_w        [T, k] fp32   output, routing weight per slot (fp32 exp; ~1e-7 relative)
 *   expert_counts [E]    int32  output, number of (token, slot) assignments per expert
 *                               (overwritten, not accumulated)
 */
int moe_route(const float* logits, const float* sel_bias, int T, int E, int k, int scoring,
              int32_t* topk_ids, float* topk_w, int32_t* expert_counts, void* stream);

/*
 * Dispatch, step 4: groups the T*k assignment rows r = t*k + j by expert. The pages name the
 * grouped expert matmul over the expert stacks (zonos2.cpp INTERNALS, "Performance": mul_mat_id
 * over the expert stacks) but not its bookkeeping; this call fixes it:
 *   expert_offsets[e] = sum_{e' < e} expert_counts[e'],  expert_offsets[E] = T*k
 *   sorted_rows[expert_offsets[e] + i] = the i-th row r (ascending r) with topk_ids[r] == e
 *   row_pos[r] = the position of row r in sorted_rows (the inverse permutation)
 *   topk_ids      [T, k]  int32  input (values must be in [0, E))
 *   expert_counts [E]     int32  input, the histogram of topk_ids (as moe_route writes it); the
 *                                kernels recount from topk_ids, so a wrong value here cannot
 *                                send a write out of bounds
 *   expert_offsets[E + 1] int32  output
 *   sorted_rows   [T * k] int32  output
 *   row_pos       [T * k] int32  output
 * All results are exact integers, identical on every call.
 */
int moe_permute(const int32_t* topk_ids, const int32_t* expert_counts, int T, int E, int k,
                int32_t* expert_offsets, int32_t* sorted_rows, int32_t* row_pos, void* stream);

/*
 * Expert FFN, steps 5-6: for every expert e and every row at position p of its group
 * (expert_offsets[e] <= p < expert_offsets[e+1]), with token t = sorted_rows[p] / k:
 *   g = w_gate[e] x[t],  u = w_up[e] x[t],  h = silu(g) * u,  expert_out[p] = w_down[e] h
 * with silu(z) = z / (1 + exp(-z)) (audio.cpp PR #1271, "Summary": SwiGLU FFN; zonos2.cpp
 * INTERNALS, "Recommended: F16 spine + K-quant experts": ffn_{gate,up,down}_exps stacks).
 *   x          [T, d]     dtype
 *   w_gate     [E, H, d]  dtype
 *   w_up       [E, H, d]  dtype
 *   w_down     [E, d, H]  dtype
 *   expert_offsets [E+1], sorted_rows [T*k]: as produced by moe_permute
 *   expert_out [T*k, d]   fp32 output, in grouped (sorted) order
 *   ws, ws_bytes          device workspace of at least moe_workspace_size(T, d, E, H, k, dtype)
 * bf16: products on MFMA with fp32 accumulation; h is rounded to fp16 (saturated at +-65504)
 * before the down matmul, which runs on fp16 operands (bf16 weights convert exactly for
 * magnitudes 2^-17..65504; smaller ones are rounded toward zero, an error below 2^-24).
 * fp32: fp32 FMA throughout.
 */
int moe_expert_ffn(const void* x, int T, int d, const void* w_gate, const void* w_up,
                   const void* w_down, int E, int H, int k, int dtype,
                   const int32_t* expert_offsets, const int32_t* sorted_rows, float* expert_out,
                   void* ws, size_t ws_bytes, void* stream);

/*
 * Combine, step 7: y[t] = sum_{j=0}^{k-1} topk_w[t, j] * expert_out[row_pos[t*k + j]], summed in
 * slot order in fp32 (zonos2.cpp INTERNALS, "Model architecture", Router row: prob-weighted sum;
 * "Notes": F32 residual stream, hence the fp32 default).
 *   expert_out [T*k, d] fp32, row_pos [T*k] int32, topk_w [T, k] fp32 -> y [T, d]
 *   y_dtype    MOE_F32 (y is float) or MOE_BF16 (y holds bf16 bits: the fp32 sum rounded once to
 *              nearest even); anything else returns MOE_ERR_UNSUPPORTED
 * Sizes: 0 <= T <= 2^24, 1 <= k <= 8, d a multiple of 4, T * k * d < 2^31. Changed in ABI 4
 * (y_dtype added).
 */
int moe_combine(const float* expert_out, const int32_t* row_pos, const float* topk_w, int T,
                int d, int k, void* y, int y_dtype, void* stream);

/* Arguments of the fused layer call. Set struct_size = sizeof(struct moe_layer_args). */
typedef struct moe_layer_args {
  uint32_t struct_size;
  int32_t T, d, E, H, k;
  int32_t dtype;             /* MOE_F32 or MOE_BF16: x and all weights                    */
  int32_t scoring;           /* enum moe_scoring                                          */
  const void* x;             /* [T, d]                                                    */
  const void* w_router;      /* [E, d]                                                    */
  const float* router_bias;  /* [E] or NULL; part of the logits (enters the weights)      */
  const float* sel_bias;     /* [E] or NULL; SELECTED_SOFTMAX ranking only                */
  const void* w_gate;        /* [E, H, d]                                                 */
  const void* w_up;          /* [E, H, d]                                                 */
  const void* w_down;        /* [E, d, H]                                                 */
  void* y;                   /* [T, d] output: fp32, or bf16 when y_dtype = MOE_BF16      */
  /* Optional outputs (NULL = not written). */
  float* logits;             /* [T, E] fp32 router logits                                 */
  int32_t* topk_ids;         /* [T, k]                                                    */
  float* topk_w;             /* [T, k]                                                    */
  int32_t* expert_counts;    /* [E]                                                       */
  /* Optional stage timing (NULL = none): an array of MOE_PROF_EVENTS hipEvent_t handles passed
     as void*, owned by the caller. [0] before routing, [1] after routing (logits, top-k,
     weights), [2] start and [3] end of the gate/up + SwiGLU kernel, [4] after the down projection
     and combine. [2] and [3] are taken by the gate/up launch itself (hipExtLaunchKernelGGL
     start/stop events), so [2] -> [3] is that kernel's duration; the others are event records
     enqueued at the stage boundary. Host launches only: a non-NULL prof_events on a stream that
     is being captured into a graph returns MOE_ERR_UNSUPPORTED with nothing enqueued. */
  void* const* prof_events;
  /* ABI 2. w_dtype = 0, or a struct_size that ends before w_dtype (MOE_LAYER_ARGS_V1_SIZE),
     means the expert weights have the activation dtype (as does w_dtype = dtype).
     w_dtype = MOE_I8: w_gate, w_up and w_down hold int8 codes in the same [E,H,d] / [E,d,H]
     layouts, and the quantisation arrays hold their fp32 row scales ([E,H], [E,H], [E,d]) as
     written by moe_quantize_rows_i8; the layer computes with the weights scale * code.
     w_dtype = MOE_Q4 (ABI 3): w_gate, w_up and w_down hold packed 4-bit codes ([E,H,d/2],
     [E,H,d/2], [E,d,H/2] bytes) and the quantisation arrays their uint32 (scale, bias) pairs
     ([E,H,d/64], [E,H,d/64], [E,d,H/64]), both as written by moe_quantize_groups_q4; the layer
     computes with the weights scale * code + bias of each group, each formed by one fp16 fused
     multiply-add (rounded to nearest) for the matrix cores (scale, bias and the gate/up products'
     bf16 token rows convert to fp16 exactly for magnitudes 2^-14..65504).
     These quantised decode paths (fewer bytes per weight: the pages run quantised expert stacks
     for decode, ZONOS2-4bit MLX card, "Performance notes" and "Quantization recipe"; zonos2.cpp
     INTERNALS, "Recommended: F16 spine + K-quant experts") need dtype = MOE_BF16 and the
     weight-streaming regime (T*k <= 2048, T*k <= 32*E, d and H multiples of 256): anything else
     returns MOE_ERR_UNSUPPORTED. Missing quantisation arrays: MOE_ERR_NULL. They must be 16-byte
     aligned.
     w_dtype = MOE_BF16_FRAG, MOE_I8_FRAG, MOE_Q4_FRAG (ABI 5): w_gate, w_up and w_down hold the
     bf16 stacks, the int8 codes or the packed 4-bit codes reordered by moe_pack_weights_frag
     (rows = E * H, K = d for gate and up; rows = E * d, K = H for down); the quantisation arrays
     as for MOE_I8 and MOE_Q4 (unchanged, row-major), not read for MOE_BF16_FRAG. dtype must be
     MOE_BF16; MOE_I8_FRAG and MOE_Q4_FRAG need the weight-streaming regime above, MOE_BF16_FRAG
     serves every shape (the grouped GEMM reads each fragment as one of its 1 KB copies). The
     result equals that of the row-major weights bit for bit. */
  int32_t w_dtype;
  const void* w_gate_scale;   /* MOE_I8: float [E, H];  MOE_Q4: uint32 [E, H, d / 64] */
  const void* w_up_scale;     /* MOE_I8: float [E, H];  MOE_Q4: uint32 [E, H, d / 64] */
  const void* w_down_scale;   /* MOE_I8: float [E, d];  MOE_Q4: uint32 [E, d, H / 64] */
  /* ABI 4. Type of y: MOE_F32 (also when struct_size ends before this field,
     MOE_LAYER_ARGS_V2_SIZE) or MOE_BF16 (the fp32 sum of the weighted expert outputs rounded once
     to nearest even). Anything else returns MOE_ERR_UNSUPPORTED. */
  int32_t y_dtype;
} moe_layer_args;

#define MOE_LAYER_ARGS_V1_SIZE offsetof(moe_layer_args, w_dtype)
#define MOE_LAYER_ARGS_V2_SIZE offsetof(moe_layer_args, y_dtype)

#define MOE_PROF_EVENTS 5

/*
 * The whole layer, steps 1-7, as one capturable sequence of kernels on `stream`:
 *   y = moe_combine(moe_expert_ffn(x, moe_permute(moe_route(moe_router_logits(x)))))
 * Routing (ids, weights, counts) equals moe_route applied to the logits this call computes
 * (write them out through `logits` to check). Internally the combine is fused into the down
 * matmul where that stays deterministic (k <= 2). ws must hold moe_workspace_size(...) bytes.
 */
int moe_layer_forward(const moe_layer_args* args, void* ws, size_t ws_bytes, void* stream);

/*
 * The fused layer for callers that cannot allocate (code under HIP graph capture, tight serving
 * loops, harnesses that forbid device allocation): moe_layer_forward with its workspace in a
 * fixed device array of the library (MOE_NOALLOC_SCRATCH_BYTES per GPU, created with the
 * library's code object on each GPU it runs on and held until the process ends) instead of a
 * caller-provided buffer. The caller still passes every input and output through `a`.
 *   - Shapes whose moe_workspace_size exceeds MOE_NOALLOC_SCRATCH_BYTES return MOE_ERR_WORKSPACE
 *     with nothing enqueued (the five model workloads of this library need at most 45 MB).
 *   - Allocates nothing: no hipMalloc, no hipFree. The first call on a device looks up the
 *     array's device address (hipGetSymbolAddress, with that device current) and keeps it; make
 *     that first call outside graph capture.
 *   - Every call on one GPU shares that GPU's array and finds the previous call's contents
 *     there (nothing in it needs clearing: every region is written before it is read). Calls
 *     that overlap in time on one GPU (different streams, or host threads racing) race on it:
 *     serialise them.
 *   - Results are identical to moe_layer_forward with its own workspace (same kernels).
 * Added in ABI 4.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)

int moe_layer_forward_noalloc(const moe_layer_args* a, void* stream);

/*
 * Symmetric per-row int8 codes of a row-major [rows, K] weight matrix (an expert stack is
 * rows = E * N rows of length K): for each row r,
 *   scales[r] = fp32(max_i |w[r,i]| / 127)                       (one IEEE round-to-nearest-even
 *   q[r,i]    = clamp(rint(fp32(w[r,i] / scales[r])), -127, 127)    division each; rint = ties to
 *                                                                   even)
 * and an all-zero row gets scale 0 and codes 0. Codes and scales are defined exactly by these
 * fp32 operations. w: device, dtype MOE_BF16 or MOE_F32; q: device int8 [rows, K]; scales: device
 * fp32 [rows]. 1 <= K, K % 16 == 0; rows >= 0 (0 is a no-op); pointers 16-byte aligned. Non-finite
 * weights are outside the contract. Asynchronous on `stream`, capturable, allocates nothing.
 * Added in ABI 2.
 */
int moe_quantize_rows_i8(const void* w, int64_t rows, int K, int dtype, int8_t* q, float* scales,
                         void* stream);

/*
 * 4-bit affine codes of a row-major [rows, K] weight matrix in groups of 64 along K (the
 * ZONOS2-4bit card quantises the experts affinely at 4 bits with group size 64, "Quantization
 * recipe"; the arithmetic below is this library's reading). For each group of 64 values w_i:
 *   lo, hi = min, max;   s = bf16(fp32(fp32(hi - lo) / 15));   b = bf16(lo)
 *   q_i    = clamp(rint(fp32(fp32(w_i - b) / s)), 0, 15)   (ties to even; s == 0 gives q_i = 0)
 * where fp32() is one IEEE round-to-nearest-even operation and bf16() rounds to nearest even.
 * The weight the layer uses is s * q_i + b.
 * Outputs (device): qpar uint32 [rows, K / 64], bf16 bits of s in the low half and of b in the
 * high half; q uint8 [rows, K / 2] in this packed order: the 64 bytes of block j (k = 128 j ..
 * 128 j + 127) are 16 little-endian uint32 words, word 4 g + c holding the codes of k = 128 j +
 * 32 c + 8 g + i, i = 0..7, with i = 2 m in bits 4 m .. 4 m + 3 and i = 2 m + 1 in bits
 * 16 + 4 m .. 19 + 4 m (g, c, m = 0..3). Each 16-byte quarter of a block is then the eight-code
 * runs one lane group of the matrix cores needs, and a shift and a mask turn two codes into
 * a pair of bf16 values.
 * w: device, dtype MOE_BF16 or MOE_F32. 128 <= K, K % 128 == 0 (MOE_ERR_SHAPE otherwise); rows >= 0
 * (0 is a no-op); pointers 16-byte aligned. Non-finite weights are outside the contract.
 * Asynchronous on `stream`, capturable, allocates nothing. Added in ABI 3.
 */
int moe_quantize_groups_q4(const void* w, int64_t rows, int K, int dtype, uint8_t* q,
                           uint32_t* qpar, void* stream);

/*
 * Fragment-major copy of an expert weight matrix (MOE_BF16_FRAG, MOE_I8_FRAG, MOE_Q4_FRAG). The
 * runtime on the pages converts checkpoints once, offline, into its own storage (zonos2.cpp
 * INTERNALS, "Converting to GGUF"); this order is the library's own. w is a row-major matrix of
 * `rows` rows with reduction length K (an expert stack is rows = E * N rows), stored as w_dtype:
 * MOE_BF16 (bf16 bits, 2 K bytes per row), MOE_I8 (int8 codes of moe_quantize_rows_i8, K bytes
 * per row) or MOE_Q4 (packed codes of moe_quantize_groups_q4, K / 2 bytes per row). out receives
 * the same bytes with each slab of 16 rows (rows 16 b .. 16 b + 15) stored as consecutive
 * 1024-byte chunks, bytes 16 l .. 16 l + 15 of chunk i (lane l = 0..63, g = l / 16) taken from row
 * 16 b + l % 16:
 *   MOE_BF16, MOE_Q4: row bytes 64 i + 16 g .. + 15 (bf16: the eight values k = 32 i + 8 g + 0..7,
 *                     the operand that lane l of a 16 x 16 x 32 matrix-core step takes; q4: the
 *                     four packed words of block i that hold k = 128 i + 32 c + 8 g + 0..7);
 *   MOE_I8:           row bytes 128 (i / 2) + 32 g + 16 (i % 2) .. + 15 (codes at those k);
 * i.e. the pieces in the order in which a wave of the decode kernels loads them, so that each load
 * instruction reads one contiguous kilobyte (bf16: also one K step's copy of 16 weight rows in the
 * prefill GEMM). Scales and (scale, bias) pairs are not reordered.
 * w, out: device, 16-byte aligned, not overlapping. rows % 16 == 0, rows >= 0 (0 is a no-op);
 * K a multiple of 32 (MOE_BF16) or 128 (codes), that multiple <= K <= 2^20; rows * K < 2^36;
 * else MOE_ERR_SHAPE. Other w_dtype: MOE_ERR_UNSUPPORTED. NULL pointers (rows > 0): MOE_ERR_NULL.
 * Exact (a reordering). Asynchronous on `stream`, capturable, allocates nothing. Added in ABI 5.
 */
int moe_pack_weights_frag(const void* w, int64_t rows, int K, int w_dtype, void* out,
                          void* stream);

/*
 * Graph ladder (serving-side decode). zonos2.cpp INTERNALS, "Performance": the decode graph is
 * captured once and replayed. A serving loop's batch width changes from step to step, so the
 * ladder captures moe_layer_forward once per bucket of batch sizes and replays the smallest bucket
 * that holds the step's tokens. Added in ABI 3.
 *
 * moe_ladder_create: `a` describes the layer at its largest batch: every token-indexed buffer (x,
 *   y, and the optional logits, topk_ids, topk_w) holds a->T rows. For bucket b the captured graph
 *   runs moe_layer_forward on the first b rows of those buffers, with every other argument of `a`
 *   (weights, biases, expert_counts, ws) unchanged; prof_events is ignored. buckets: n_buckets
 *   (1..MOE_LADDER_MAX_BUCKETS) strictly ascending sizes in 1..a->T. ws must hold
 *   moe_workspace_size(a->T, ...) bytes. Every buffer must stay alive and in place until
 *   moe_ladder_destroy. `stream` must be a real stream (not NULL) that is not being captured; the
 *   call captures on it and enqueues no work. Unlike every other entry point it allocates: host
 *   memory and the graphs' resources; it is not itself capturable. Errors: MOE_ERR_NULL,
 *   MOE_ERR_SHAPE (buckets), MOE_ERR_UNSUPPORTED (stream), any error moe_layer_forward returns for
 *   a bucket (nothing is kept), MOE_ERR_HIP (capture or instantiation failed).
 * moe_ladder_run: replays, on `stream`, the graph of the smallest bucket b >= T (1 <= T <= the
 *   largest bucket, else MOE_ERR_SHAPE). Rows T..b-1 are computed as extra tokens from whatever x
 *   holds there (their outputs go to rows T..b-1 of y and of the optional outputs); rows below T
 *   are exactly what moe_layer_forward on the first T rows gives whenever both calls take the same
 *   kernel path. expert_counts (if given) counts the first T rows only: when b > T a small kernel
 *   recounts it from their ids after the replay. *bucket_out (if not NULL) receives b.
 *   Capturable (a graph launch, and that kernel).
 * moe_ladder_destroy: releases the ladder (NULL is a no-op); the caller's stream work using it must
 *   have completed.
 */
#define MOE_LADDER_MAX_BUCKETS 256

typedef struct moe_graph_ladder moe_graph_ladder;

int moe_ladder_create(const moe_layer_args* a, const int32_t* buckets, int n_buckets, void* ws,
                      size_t ws_bytes, void* stream, moe_graph_ladder** out);
int moe_ladder_run(const moe_graph_ladder* ladder, int T, void* stream, int32_t* bucket_out);
void moe_ladder_destroy(moe_graph_ladder* ladder);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
