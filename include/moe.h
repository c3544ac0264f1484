/*
 * moe.h: C ABI of the MI355X (gfx950) fine-grained-quantized MoE experts forward.
 *
 * The operation follows these pages (cited by title and section):
 *  [P-grouped]  "grouped_mm experts dispatch does not support
 *               activation_scheme='static'", sections "What it means" and
 *               "Source": the grouped experts forward flattens the (token, slot)
 *               pairs, sorts them by expert id, gathers each pair's token row,
 *               quantizes activations dynamically per block, runs the grouped
 *               GEMMs, then zeroes sentinel rows, weights each slot's output and
 *               sums the k slots of a token with a deterministic reshape+sum
 *               (not an atomic index_add_) before casting back to bf16.
 *  [P-mega]     "DeepGEMM Mega MoE requires a `process_group` for the EP group",
 *               the forward's docstring: top_k_index holds global expert ids,
 *               -1 marks a skipped slot; gate_up_proj / down_proj are the L1 / L2
 *               weights with UE8M0 scale factors, transformed once; an optional
 *               swiglu_limit clamps the SwiGLU (absent means unclamped).
 *  [P-fp4]      "DeepGEMM Mega MoE requires FP4-packed expert weights
 *               (dtype=int8)", section "Source": FP4 weights come packed in int8.
 *  [P-devices]  "DeepGEMM experts selected on a model spanning multiple CUDA
 *               devices", the record's source: the forward refuses a multi-device
 *               model and non-bf16 hidden states before any kernel work, and
 *               picks the nn or nt weight layout.
 *  [P-grouped] also names the static activation scheme: precomputed activation
 *               scales that the pages' eager path consumes and their grouped
 *               path refuses ("What it means", "Example fix"); this library
 *               serves it (moe_quant_act_static, moe_options.act_scales).
 *
 * Conventions for every call:
 *  - Pointers marked "device" are device memory on the device current for
 *    `stream`; the caller owns every buffer.  Nothing here allocates device
 *    memory, frees it, or synchronizes the host: every call validates its
 *    arguments on the host, enqueues its kernels on `stream` and returns.
 *  - Inputs are read-only.  Outputs must not alias inputs.
 *  - Validation failures return before anything is enqueued; the text of the
 *    last failure on the calling thread is available from moe_last_error().
 *  - T (tokens), k (slots per token), E (local experts), H (hidden size) and
 *    I (expert intermediate size) are as in the forward; S = T * k slots.
 *  - Shapes: H and I must be multiples of 128.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h> /* hipStream_t only */

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,        /* a required pointer is NULL */
  MOE_ERR_SHAPE = 2,       /* a size is out of range or not a multiple of the block */
  MOE_ERR_DTYPE = 3,       /* an argument has the wrong element type (the pages: ValueError on non-bf16 input) */
  MOE_ERR_UNSUPPORTED = 4, /* a request this library does not serve (aliasing, static scales on bf16 experts) */
  MOE_ERR_WORKSPACE = 5,   /* workspace missing or smaller than the matching *_workspace() size */
  MOE_ERR_ARCH = 6,        /* the stream's device is not gfx950 */
  MOE_ERR_DEVICE = 7,      /* a pointer lives on another device than the stream */
  MOE_ERR_HIP = 8          /* the HIP runtime reported an error while enqueueing */
} moe_status;

/* Quantization formats.
 * MOE_FMT_FP8_B128: activations e4m3 (OCP e4m3fn) with one fp32 scale per 1x128
 *   block along the row; weights e4m3 with one fp32 scale per 128x128 block.
 * MOE_FMT_MXFP8A_MXFP4W: activations e4m3 with one UE8M0 scale byte per 1x32
 *   block; weights e2m1 packed two per byte along K (even k in the low nibble)
 *   with one UE8M0 byte per 1x32 block along K.  A UE8M0 byte b means 2^(b-127).
 * In both, a dequantized value is code value times its block scale.
 * MOE_FMT_BF16: the unquantized experts the pages fall back to ([P-devices]:
 *   experts_implementation='grouped_mm'): bf16 activations and bf16 weights,
 *   no scales, fp32 accumulation; h = SwiGLU(g, u) is rounded once to bf16 and
 *   is the down projection's operand.  The forward needs T*H and T*k*I below
 *   2^31 elements (MOE_ERR_SHAPE otherwise). */
typedef enum moe_format { MOE_FMT_FP8_B128 = 0, MOE_FMT_MXFP8A_MXFP4W = 1, MOE_FMT_BF16 = 2 } moe_format;

/* Weight layouts accepted by moe_prepare_weights: nt stores each expert's weight
 * as [N, K] (rows are output features), nn as [K, N]; the pages' forward picks
 * between the two grouped matmuls by this flag ([P-devices]). */
typedef enum moe_layout { MOE_LAYOUT_NT = 0, MOE_LAYOUT_NN = 1 } moe_layout;

const char* moe_status_string(moe_status s);
/* Detail text of the last failed call on this thread ("" when none). */
const char* moe_last_error(void);

/* ------------------------------------------------------------ route sort --
 * Sorts the S = T*k flat slots s = t*k + j by expert ([P-grouped], "Source":
 * the flattened expert ids are sorted and the rows gathered by perm // k).
 * key(s) = top_k_index[s] - expert_begin when that lies in [0, E), otherwise
 * the slot is skipped and gets the sentinel key E ([P-mega]: -1 marks a skipped
 * slot; ids outside this GPU's range are treated the same way).  Sentinels sort
 * after every valid slot and ties keep ascending s, so the result is unique.
 *
 *  top_k_index     device int32 [T*k], global expert ids.
 *  sorted_slot     device int32 [T*k] out: the flat slot at each sorted row.
 *  expert_offsets  device int32 [E+1] out: number of slots with key < e;
 *                  expert e owns sorted rows [offsets[e], offsets[e+1]) and
 *                  offsets[E] is the number of valid slots.
 *  slot_pos        device int32 [T*k] out, may be NULL: inverse of sorted_slot.
 *  invalid_count   device int32 [1] out, may be NULL: number of ids that are
 *                  neither -1 nor inside [expert_begin, expert_begin + E).
 *  ws / ws_bytes   device workspace of at least moe_route_sort_workspace()
 *                  bytes (per-chunk histograms; 0 bytes, and ws may be NULL,
 *                  below 16384 slots).  Its contents are scratch.
 * Limits: 0 <= T, 1 <= k <= 64, 1 <= E <= 512, T*k < 2^31, expert_begin >= 0
 * (global ids are non-negative, so -1 is never a local expert). */
size_t moe_route_sort_workspace(int32_t T, int32_t k, int32_t E);
moe_status moe_route_sort(const int32_t* top_k_index, int32_t T, int32_t k, int32_t E, int32_t expert_begin,
                          int32_t* sorted_slot, int32_t* expert_offsets, int32_t* slot_pos,
                          int32_t* invalid_count, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------- router + route sort --
 * The router step in front of the experts forward, fused with the route sort.
 * The pages hand the router's output to the experts untouched, as global
 * expert ids with unmasked weights ("deepgemm_megamoe EP implementation for
 * DeepGEMM Mega MoE", PR #49606: "How it runs" and the parallel-style table);
 * the router of the layers this forward is shaped on (Mixtral, Qwen3-MoE) is a
 * softmax over the expert logits, the k most probable experts, and their
 * probabilities renormalised to sum 1.  Per token t:
 *   ids:     the k largest of router_logits[t, 0..n_experts), compared as fp32
 *            values, in descending order, the lower id first among equal
 *            logits (softmax is increasing, so these are the k most probable);
 *   weights: p_e = exp(l_e - max_e' l_e') / sum over all e' of the same terms;
 *            top_k_weights[t, j] = p of ids[t, j], divided by the sum of the k
 *            selected p when `renormalize` is nonzero.  Computed in fp32 (the
 *            difference l - max rounded once, exp accurate to about 1 ulp,
 *            sums in lane order): a weight agrees with an exact computation
 *            to a relative (n_experts + 4 + 2 (max - min of the token's
 *            logits)) * 2^-24; the ids agree exactly.
 * Logits must be finite (not checked).
 *
 *  router_logits   device float [T, n_experts], row-major.
 *  top_k_index     device int32 [T, k] out: the chosen global ids.
 *  top_k_weights   device float [T, k] out.
 *  E, expert_begin, sorted_slot, expert_offsets, slot_pos, invalid_count, ws:
 *                  as in moe_route_sort, applied to the chosen ids (ids
 *                  outside [expert_begin, expert_begin + E) are sentinels).
 *                  expert_offsets NULL runs the router alone (sorted_slot
 *                  and slot_pos must then be NULL too; E and ws are unused).
 * Up to 16 tokens of at most 128 experts (and fewer than 16384 slots), the
 * router and the sort run in one launch; otherwise the router is a launch of
 * its own.
 * Limits: 1 <= n_experts <= 512, 1 <= k <= min(64, n_experts); the rest as in
 * moe_route_sort. */
size_t moe_route_topk_workspace(int32_t T, int32_t k, int32_t E);
moe_status moe_route_topk(const float* router_logits, int32_t T, int32_t n_experts, int32_t k, int32_t renormalize,
                          int32_t* top_k_index, float* top_k_weights, int32_t E, int32_t expert_begin,
                          int32_t* sorted_slot, int32_t* expert_offsets, int32_t* slot_pos, int32_t* invalid_count,
                          void* ws, size_t ws_bytes, hipStream_t stream);

/* --------------------------------------------------- activation quantization --
 * Dynamic per-block quantization of bf16 rows ([P-grouped], "What it means":
 * activations are quantized dynamically per block).  Per block of B = 128
 * (FP8_B128) or 32 (MX) elements of a row:
 * amax = max|x|; FP8_B128: s = max(amax, 1e-4f) / 448 in fp32 and
 * code = e4m3(x / s) with an IEEE fp32 division; MX: e = ceil(log2(max(amax,
 * 1e-4f) / 448)) read exactly from the fp32 bits, scale byte e + 127 and
 * code = e4m3(x * 2^-e).  e4m3() rounds to nearest even and saturates at 448.
 *
 * Activation layout used by this library ("K-block-major"): a [rows, K] matrix
 * of codes is stored as K/128 planes of [rows][128] bytes, i.e. byte
 * (row, k) lives at (k / 128) * rows * 128 + row * 128 + k % 128; its scales are
 * float [K/128][rows] (FP8_B128) or uint8 [K/128][rows][4] (MX: the four UE8M0
 * bytes of a row's 128-wide block, in K order).
 *
 *  x       device bf16 bit patterns [rows, H], row-major.
 *  codes   device uint8 out, K-block-major [H/128][rows][128].
 *  scales  device out: float [H/128][rows] (FP8_B128) or uint8 [H/128][rows][4] (MX). */
moe_status moe_quant_act(const uint16_t* x, int32_t rows, int32_t H, moe_format fmt, uint8_t* codes, void* scales,
                         hipStream_t stream);

/* Static per-block quantization: the activation scheme whose scales are
 * precomputed ([P-grouped], "What it means" and "Example fix": the static
 * scheme implies pre-computed activation scales, which the pages' eager path
 * consumes).  The caller's block scales replace the amax pass; the encoding is
 * moe_quant_act's: FP8_B128 code = e4m3(x / s) with an IEEE fp32 division, MX
 * code = e4m3(x * 2^-(b - 127)); e4m3() rounds to nearest even and saturates
 * at 448, so |x| >= 448 s gives the largest code of x's sign.
 *
 *  act_scales  device, read-only: FP8_B128 float, MX uint8 UE8M0 bytes; row t's
 *              H/128 (FP8_B128) or H/32 (MX) block scales start at element
 *              t * row_stride.  row_stride 0 gives every row the same scales
 *              (one row of block scales, e.g. a per-tensor scale repeated);
 *              otherwise row_stride >= H/128 (H/32).  FP8 scales must be
 *              finite and > 0 and MX bytes < 255 (not checked: a zero or
 *              non-finite scale gives unspecified codes).
 *  codes, scales  out, as moe_quant_act (the scales are the caller's, copied
 *              into the K-block-major layout the grouped GEMM reads). */
moe_status moe_quant_act_static(const uint16_t* x, int32_t rows, int32_t H, moe_format fmt, const void* act_scales,
                                int32_t row_stride, uint8_t* codes, void* scales, hipStream_t stream);

/* --------------------------------------------------------- expert weights --
 * Descriptor of one layer's prepared expert weights (filled by
 * moe_prepare_weights; the code arrays are in the library's tiled layout and
 * are not meant to be read by the caller):
 *  w13 / w13_scale  gate_up weight codes (tiled) and its scales,
 *                   FP8_B128: float [E, 2I/128, H/128].
 *  w2 / w2_scale    down weight codes (tiled) and its scales,
 *                   FP8_B128: float [E, H/128, I/128].
 *                   MX: the scales are tiled like the codes.
 * All four are device pointers that must stay valid while the descriptor is used. */
typedef struct moe_weights {
  moe_format fmt;
  int32_t E, H, I;
  const uint8_t* w13;
  const void* w13_scale;
  const uint8_t* w2;
  const void* w2_scale;
} moe_weights;

/* One-shot weight preparation ([P-mega]: both weight pairs are transformed
 * together once, before the first forward, into the kernel's own layout).
 * Inputs, device memory, as the checkpoint stores them:
 *  layout NT: gate_up [E, 2I, H] (rows [0, I) gate, [I, 2I) up), down [E, H, I];
 *  layout NN: gate_up [E, H, 2I], down [E, I, H] (each expert's weight transposed).
 *  FP8_B128: uint8 e4m3 codes; scales float per 128x128 block, [E, 2I/128, H/128]
 *  and [E, H/128, I/128] for NT, transposed ([E, H/128, 2I/128], [E, I/128, H/128])
 *  for NN.
 *  MX (NT only): gate_up packed e2m1 [E, 2I, H/2] (even k in the low nibble),
 *  down packed [E, H, I/2]; UE8M0 scales uint8 [E, 2I, H/32] and [E, H, I/32].
 *  BF16: bf16 values, gate_up [E, 2I, H] and down [E, H, I] for NT, [E, H, 2I]
 *  and [E, I, H] for NN; both scale pointers are ignored and may be NULL (the
 *  descriptor's are NULL).
 * The tiled copy goes to `prepared` (device, at least moe_prepared_weights_size()
 * bytes, owned by the caller); `out` is filled on the host.  Enqueued on
 * `stream`.  Weight quantization itself is offline (the checkpoint's). */
size_t moe_prepared_weights_size(moe_format fmt, int32_t E, int32_t H, int32_t I);
moe_status moe_prepare_weights(moe_format fmt, moe_layout layout, int32_t E, int32_t H, int32_t I,
                               const void* gate_up, const void* gate_up_scale, const void* down,
                               const void* down_scale, void* prepared, size_t prepared_bytes, moe_weights* out,
                               hipStream_t stream);

/* ----------------------------------------------------------- grouped GEMM --
 * For every expert e and sorted row r in [offsets[e], offsets[e+1]):
 *   C[r, n] = sum_i A[a_row(r), i] * B[e, n, i]      (n < N, i < K)
 * with both operands dequantized (code times block scale), products exact and
 * sums in fp32.  B is one weight of a prepared moe_weights: which = 0 the
 * gate_up weight (N = 2I, K = H), which = 1 the down weight (N = H, K = I).
 * a_row(r) = a_row_index[r] / a_row_divisor, or r when a_row_index is NULL (the
 * row gather of [P-grouped], "Source").  A is K-block-major (see moe_quant_act)
 * with a_rows rows per plane.  Then one epilogue:
 *  MOE_EPI_STORE_F32         c_f32[r, n] = C[r, n]           (fp32 [max_rows, N], row-major)
 *  MOE_EPI_SWIGLU_QUANT      which = 0: g = C[r, n], u = C[r, I + n] for n < I;
 *                            with a limit L, g = min(g, L), u = clamp(u, -L, L);
 *                            h = silu(g) * u, quantized per block along I with the
 *                            activation rule into h_codes (K-block-major
 *                            [I/128][max_rows][128]) and h_scales (float
 *                            [I/128][max_rows] or uint8 [I/128][max_rows][4]).
 *  MOE_EPI_WEIGHTED_SCATTER  slot = slot_of_row[r]:
 *                            slot_out[slot, n] = bf16(top_k_weights[slot] * C[r, n])
 *                            (bf16 [S, N], row-major).
 * Rows at and beyond offsets[E] are not written.  max_rows bounds offsets[E]
 * (normally T*k).
 * a_scales_sorted (optional, may be NULL): the same activation scales laid out
 * by sorted row, [K/128][max_rows] floats or [K/128][max_rows][4] UE8M0 bytes,
 * row r holding the scales of A row a_row(r).  The 256-row tiled paths then read
 * it instead of a_scales (consecutive addresses instead of a gather); a_scales
 * stays required, and the few-rows FP8 path reads it.  The forward builds such
 * a copy when moe_forward_sorts_scales() says so.
 * MOE_FMT_BF16 weights: A is bf16 [a_rows, K] row-major (not K-block-major),
 * below 4 GiB, and a_scales is ignored; the SwiGLU epilogue writes h as bf16
 * [max_rows, I] row-major into h_codes (h_scales ignored). */
typedef enum moe_epilogue {
  MOE_EPI_STORE_F32 = 0,
  MOE_EPI_SWIGLU_QUANT = 1,
  MOE_EPI_WEIGHTED_SCATTER = 2
} moe_epilogue;

typedef struct moe_gemm_args {
  const moe_weights* weights;
  int32_t which; /* 0 = gate_up, 1 = down */
  int32_t max_rows;
  const uint8_t* a_codes;
  const void* a_scales;
  int32_t a_rows;             /* rows per K-block plane of A */
  const int32_t* a_row_index; /* may be NULL */
  int32_t a_row_divisor;      /* >= 1 */
  const int32_t* expert_offsets; /* [E+1] */
  moe_epilogue epilogue;
  float* c_f32;
  uint8_t* h_codes;
  void* h_scales;
  int32_t has_swiglu_limit;
  float swiglu_limit;
  uint16_t* slot_out;
  const float* top_k_weights;
  const int32_t* slot_of_row;
  /* May be NULL (tiles are then taken in a fixed round-robin order).  Else
   * device memory of MOE_TILE_COUNTERS_BYTES, 8-byte aligned (MOE_ERR_SHAPE
   * otherwise), all zero before the launch:
   * workgroups then take tiles dynamically from atomic counters in it, and the
   * launch leaves it zero again.  Two launches in flight at once must not share
   * it. */
  int32_t* tile_counters;
  const void* a_scales_sorted; /* may be NULL, see above */
} moe_gemm_args;

#define MOE_TILE_COUNTERS_BYTES 1024

moe_status moe_grouped_gemm(const moe_gemm_args* args, hipStream_t stream);

/* ---------------------------------------------------- fused experts forward --
 * Whether moe_experts_forward, for T tokens of k slots in format fmt, copies
 * the activation scales by sorted row and hands that copy to its gate_up GEMM
 * (a_scales_sorted): 1 or 0, no side effects.  A caller timing that GEMM alone
 * uses it to launch it the way the forward does. */
int32_t moe_forward_sorts_scales(int32_t T, int32_t k, moe_format fmt);

/*
 * The whole path in one call ([P-grouped] and [P-mega]): route sort, activation
 * quantization, gate_up grouped GEMM with the SwiGLU (+ optional clamp) and h
 * quantization fused into its epilogue, down grouped GEMM with the routing
 * weight applied in its epilogue, and the deterministic per-token sum over the
 * k slots in ascending j.  Skipped slots are never computed and contribute
 * exactly zero whatever their weight (NaN included).
 *
 *  w               prepared weights (moe_prepare_weights).
 *  hidden_states   device bf16 [T, H].
 *  top_k_index     device int32 [T, k], global expert ids, -1 = skipped.
 *  top_k_weights   device float [T, k] (unmasked routing weights).
 *  opt             may be NULL (no clamp, expert_begin 0).
 *  out             device bf16 [T, H] out.
 *  ws / ws_bytes   device workspace of at least moe_experts_forward_workspace().
 * T == 0 returns MOE_OK with nothing enqueued.  Limits: 1 <= k <= 64 and, for
 * the quantized formats, T*k*128 < 2^31 (the GEMMs address each 128-wide K
 * plane of their row operands with 32-bit offsets; the bf16 limits are given
 * with MOE_FMT_BF16); MOE_ERR_SHAPE otherwise. */
typedef struct moe_debug {
  /* Optional device copies of intermediates, for parity checks; each may be NULL. */
  int32_t* sorted_slot;    /* [T*k] */
  int32_t* expert_offsets; /* [E+1] */
  uint8_t* act_codes;      /* K-block-major [H/128][T][128] */
  void* act_scales;        /* float [H/128][T] or uint8 [H/128][T][4] */
  /* The quantized SwiGLU output h (the down projection's operand), by sorted
   * row: K-block-major codes [I/128][T*k][128] and scales float [I/128][T*k]
   * or uint8 [I/128][T*k][4].  Only rows [0, expert_offsets[E]) are defined;
   * sorted row r belongs to flat slot sorted_slot[r].  Not written for
   * MOE_FMT_BF16. */
  uint8_t* h_codes;
  void* h_scales;
} moe_debug;

typedef struct moe_options {
  int32_t has_swiglu_limit;
  float swiglu_limit;    /* must be finite and > 0 when has_swiglu_limit */
  int32_t expert_begin;  /* global id of local expert 0, >= 0 */
  /* Nonzero: the static activation scheme.  hidden_states is quantized with
   * the caller's block scales act_scales (laid out as in moe_quant_act_static,
   * row t = token t, stride act_scales_row_stride) instead of its own block
   * amax; h, the down projection's operand, stays dynamic (the scheme gives
   * scales for the layer's input only).  Quantized formats only:
   * MOE_ERR_UNSUPPORTED for MOE_FMT_BF16, MOE_ERR_NULL without act_scales,
   * MOE_ERR_SHAPE for a stride below one row. */
  int32_t static_activation_scales;
  int32_t* invalid_count; /* device int32 [1], may be NULL */
  moe_debug* debug;       /* may be NULL */
  const void* act_scales;        /* device: float (FP8_B128) or uint8 (MX) block scales */
  int32_t act_scales_row_stride; /* elements between consecutive tokens' rows; 0 = one row for all */
} moe_options;

size_t moe_experts_forward_workspace(int32_t T, int32_t k, const moe_weights* w);
moe_status moe_experts_forward(const moe_weights* w, const uint16_t* hidden_states, const int32_t* top_k_index,
                               const float* top_k_weights, int32_t T, int32_t k, const moe_options* opt,
                               uint16_t* out, void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------ forward without allocation --
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the fused
 * forward above, with its workspace taken from a scratch array the library
 * holds in device memory, MOE_NOALLOC_SCRATCH_BYTES per GPU, for the life of
 * the process (each GPU the library runs on holds its own copy).  The caller
 * still passes the inputs and the output; the call allocates and frees
 * nothing.  A forward whose moe_experts_forward_workspace() exceeds
 * MOE_NOALLOC_SCRATCH_BYTES is refused with MOE_ERR_WORKSPACE (64 MiB holds,
 * for example, a 64-token Qwen3-MoE-shaped decode batch or 256 tokens of a
 * DeepSeek-V3-shaped layer).  Every call on a GPU shares that GPU's scratch:
 * calls that overlap on one GPU (on different streams) race and corrupt each
 * other's results; calls on one stream are ordered and safe.  Arguments,
 * results and errors are those of moe_experts_forward. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status moe_experts_forward_noalloc(const moe_weights* w, const uint16_t* hidden_states,
                                       const int32_t* top_k_index, const float* top_k_weights, int32_t T, int32_t k,
                                       const moe_options* opt, uint16_t* out, hipStream_t stream);

/* The same forward starting one step earlier, from the router's logits: the
 * router of moe_route_topk chooses each token's k experts among n_experts
 * (global ids) and their weights, writes them to top_k_index / top_k_weights
 * (device int32 / float [T, k], outputs owned by the caller), and the forward
 * above then runs on them.  Small batches route, sort and quantize in one
 * launch.  The workspace is moe_experts_forward_workspace(T, k, w).  The
 * outputs must not alias each other or the inputs. */
moe_status moe_experts_forward_from_logits(const moe_weights* w, const uint16_t* hidden_states,
                                           const float* router_logits, int32_t T, int32_t n_experts, int32_t k,
                                           int32_t renormalize, const moe_options* opt, int32_t* top_k_index,
                                           float* top_k_weights, uint16_t* out, void* ws, size_t ws_bytes,
                                           hipStream_t stream);

/* ------------------------------------------------------ measurement utility --
 * Not a step of the forward: the rate at which the matrix cores issue the MFMA
 * forms the grouped GEMMs use, with random operands held in registers (no
 * memory traffic), one workgroup of 8 waves on every CU, each wave running
 * `iters` rounds of 16 independent MFMAs (8 for kind 4), over four rotating
 * operand sets.  It exists so that each GEMM can be
 * priced against the rate its own operand types reach on the device; the
 * published peaks give FP8 and FP4 rates for matching operands only.
 *  kind 0: e4m3 x e4m3 16x16x128, accumulating in the MFMA;
 *  kind 1: e2m1 x e4m3 16x16x128 with per-lane UE8M0 scales (the MX GEMM's form);
 *  kind 2: e2m1 x e2m1 16x16x128 with per-lane UE8M0 scales;
 *  kind 3: bf16 16x16x32;
 *  kind 4: e4m3 x e4m3 16x16x128 into a fresh accumulator, then the fp32
 *          promotion acc += P * s (the FP8 GEMM's form).
 * Outputs (host): *tflops, the achieved dense TFLOP/s (2 flops per MAC), and
 * *sclk_ghz, the mean shader clock the probe ran at (shader-clock ticks over
 * the 100 MHz real-time counter, per workgroup).  Allocates and frees its own
 * device scratch and waits for the stream (a blocking call).  Errors:
 * MOE_ERR_NULL (NULL output), MOE_ERR_UNSUPPORTED (kind outside 0..4),
 * MOE_ERR_SHAPE (iters outside [1, 2^24]), device and HIP errors as elsewhere. */
moe_status moe_probe_mfma_rate(int32_t kind, int32_t iters, double* tflops, double* sclk_ghz, hipStream_t stream);

/* Clock stamps (a measurement utility, not a step of the forward): enqueues on
 * `stream` n one-wave workgroups; workgroup i writes three uint64 values to
 * stamps[3 i], stamps[3 i + 1], stamps[3 i + 2]: the compute unit it ran on
 * (XCD id * 256 + bits 8-15 of the hardware-id register: the shader engine,
 * array and CU ids), that unit's shader-clock counter and the device's 100 MHz
 * real-time counter.  Two calls on one stream bracket the work enqueued
 * between them: for a unit stamped in both, the difference of its shader-clock
 * counters over the difference of the real-time counters, times 0.1 GHz, is
 * its mean shader clock over that span (the clock the GEMMs ran at under the
 * chip's power limit).  The counters of different units are not aligned, and
 * they follow the actual clock, which drops to its idle level while there is
 * no work, so a span should hold back-to-back kernels only.  stamps: device
 * memory of 3 n uint64 on the stream's device, written asynchronously (read
 * it once the stream has passed the call).  n: 1..4096; 1024 stamp most units
 * of the 256-CU part.  Allocates nothing and does not block.  Errors: MOE_ERR_NULL
 * (stamps NULL), MOE_ERR_SHAPE (n out of range), MOE_ERR_DEVICE (stamps not on
 * the stream's device), HIP errors as elsewhere. */
moe_status moe_clock_stamp(uint64_t* stamps, int32_t n, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
