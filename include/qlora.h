/*
 * qlora.h -- C ABI of libqlora.so: the LoRA linear layer over a frozen,
 * block-quantized base weight, for AMD Instinct MI355X (gfx950).
 *
 * What is computed (Surogate README page, "LoRA & QLoRA" capability row:
 * adapters over an FP8 / NF4 quantized base; Soup page, opening paragraph:
 * the frozen base is read and never written; GGUF-recipe page, "How it
 * works": the base stays compressed during computation and LoRA uses fast
 * backward formulas):
 *
 *   forward   y  = x . deq(W)^T + s . (x . A^T) . B^T,     s = alpha / r
 *   backward  dX = dY . deq(W) + s . (dY . B) . A
 *             dA = s . (dY . B)^T . x
 *             dB = s . dY^T . (x . A^T)
 *
 * Conventions for every call below.
 *   - Shapes follow nn.Linear: W [N, K] (N = out_features, K = in_features),
 *     x [M, K], y and dY [M, N], A [r, K], B [N, r], U = x.A^T [M, r].
 *     All matrices are row-major and dense (row stride = number of columns).
 *   - bf16 tensors are passed as uint16_t bit patterns; fp32 as float.
 *   - "dev" pointers are device (HBM) pointers on the current HIP device;
 *     "host" pointers are ordinary host memory.  The caller owns every
 *     buffer; the library never allocates inside quant_pack, qlora_linear_fwd
 *     or qlora_linear_bwd (scratch comes in through ws / ws_bytes).
 *   - stream is a hipStream_t passed as void* (NULL = the null stream).  Calls
 *     enqueue work and return; buffers must stay alive until the stream has
 *     passed the work.  Argument errors are reported synchronously and
 *     nothing is enqueued.  A device fault surfaces at the caller's next
 *     synchronize and as QL_EHIP from the next library call.
 *   - Device pointers must be 16-byte aligned; M, N, K >= 1 (M may be 0:
 *     then nothing is launched), K and N multiples of the format's block
 *     (64 for NF4, 32 otherwise), r in {8, 16, 32}.
 *   - Size limits (the kernels address memory through 32-bit buffer
 *     offsets): N and K at most QL_MAX_FEATURES and the codes array of a
 *     weight below 2 GiB; larger shapes are refused with QL_EUNSUPPORTED
 *     (by every call that takes a weight or a shape, quant_pack included).
 *   - The quantized base is const: no call writes codes or scales.
 *   - Results do not depend on pointer values, only on shapes and data
 *     (fixed launch configuration and fixed reduction order per shape), so
 *     two calls on equal inputs give bitwise equal outputs.
 *   - Return value: QL_OK (0) or a negative QL_E* code; ql_last_error()
 *     gives a message for the calling thread.
 */
#ifndef QLORA_H
#define QLORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- status */
#define QL_OK 0
#define QL_EINVAL (-1)        /* bad argument: null, misaligned, shape      */
#define QL_EUNSUPPORTED (-2)  /* valid but not implemented (format, rank)   */
#define QL_EWORKSPACE (-3)    /* ws_bytes below qlora_workspace_bytes()     */
#define QL_EHIP (-4)          /* a HIP runtime call failed                  */
#define QL_ENONFINITE (-5)    /* quant_pack saw NaN or Inf in W             */
#define QL_ESTATE (-6)        /* stream-pool misuse                         */
#define QL_EOVERFLOW (-7)     /* quant_pack: a Q4_0 scale overflows fp16    */

/* largest N or K a weight may have (see the size limits above) */
#define QL_MAX_FEATURES 524288

/* ---------------------------------------------------------------- formats
 * 4-bit code layout (Q4_0 and NF4): codes are u8 [N, K/2]; each row is cut
 * into groups of 32 consecutive elements stored in 16 bytes, byte j of a
 * group holding element j in its low nibble and element j + 16 in its high
 * nibble.  Scales are a separate array.
 *
 * QL_FMT_Q4_0      legacy-GGUF-style 4-bit blocks of 32 along K (the GGUF
 *                  page's base format): scales fp16 [N, K/32],
 *                  d = fp16(absmax / 7), code q = clamp(rint(w/d) + 8, 0, 15)
 *                  (ties to even), value (q - 8) * d; a zero block stores 8.
 * QL_FMT_NF4       NormalFloat-4 (QLoRA paper, "4-bit NormalFloat"; the NF4
 *                  base named on the Surogate and Soup pages): blocks of 64
 *                  along K, scales fp32 [N, K/64] = block absmax, code =
 *                  nearest of 16 normal-quantile levels (a value equal to a
 *                  decision threshold takes the lower code), value c[q] * a;
 *                  a zero block stores 7.  No double quantization.
 * QL_FMT_FP8_E4M3  OCP E4M3FN codes u8 [N, K] (the Surogate FP8 recipe's base
 *                  format) with one fp32 scale s = absmax / 448; code =
 *                  E4M3(w / s) nearest even, saturating; value E4M3(q) * s.
 * QL_FMT_MXFP4     OCP Microscaling MXFP4 (the FP4 base behind the Surogate
 *                  pages' NVFP4 / MXFP4 recipes, whose definition the pages
 *                  leave to the OCP specification): blocks of 32 along K, one
 *                  E8M0 scale byte e per block (scales u8 [N, K/32]) standing
 *                  for X = 2^(e - 127), e - 127 = floor(log2 absmax) - 2
 *                  clamped to [-127, 127] (a zero block stores e = 0); element
 *                  code = E2M1(w / X) (1 sign, 2 exponent bits with bias 1, 1
 *                  mantissa bit; nearest even, saturating to +-6; a negative
 *                  value that rounds to zero keeps its sign); value
 *                  E2M1(q) * X, exact in fp32 and in bf16.  Codes are
 *                  pair-packed, unlike the two formats above: byte i of a row
 *                  holds element 2i in its low nibble and element 2i + 1 in
 *                  its high nibble (u8 [N, K/2]).  e = 255 is never written
 *                  and decodes to NaN.
 * QL_FMT_Q8_0      the 8-bit member of the legacy GGUF block family (the
 *                  GGUF page's Q8_0 base, whose layout the page does not
 *                  give): blocks of 32 along K, scales fp16 [N, K/32],
 *                  d = fp16(absmax / 127), code q = clamp(rint(w/d), -127,
 *                  127) (ties to even) stored as a two's complement byte, one
 *                  per element (u8 [N, K]); value q * d; a zero block stores
 *                  d = 0 and codes 0.
 * QL_FMT_NVFP4     NVFP4 (the FP4 format of the Surogate pages' Blackwell
 *                  recipe, named there as "NVFP4 (E2M1)" and not defined;
 *                  NVIDIA's published structure): E2M1 codes in blocks of 16
 *                  along K, one E4M3 scale byte per block and one fp32
 *                  scale per tensor.  g = fl32(amax / 2688) (2688 = 6 * 448);
 *                  block scale byte sb = E4M3(fl32(fl32(amax_b / 6) / g)),
 *                  nearest even, saturating at 448 (0 when g = 0); block
 *                  decode scale X = fl32(E4M3(sb) * g); element code = the
 *                  E2M1 value nearest to the exact quotient w / X (ties to
 *                  the even mantissa, saturating to +-6, sign bit from w;
 *                  0 when X = 0); value fl32(E2M1(q) * X).  Codes u8
 *                  [N, K/2] in the split-nibble groups of 32 of Q4_0 and
 *                  NF4 (a group's low nibbles are one block of 16, its high
 *                  nibbles the next).  scales: 16 + N K / 16 bytes -- g as
 *                  fp32 at byte 0, zero bytes 4..15, then the E4M3 bytes
 *                  u8 [N, K/16] from byte 16.  K must be a multiple of 32.
 */
#define QL_FMT_Q4_0 1
#define QL_FMT_NF4 2
#define QL_FMT_FP8_E4M3 3
#define QL_FMT_MXFP4 4
#define QL_FMT_Q8_0 5
#define QL_FMT_NVFP4 6

/* workspace query operations */
#define QL_OP_PACK 0
#define QL_OP_FWD 1
#define QL_OP_BWD 2

/* A packed, frozen base weight (all pointers dev, read-only). */
typedef struct ql_qweight {
  int32_t format;        /* QL_FMT_*                                        */
  int32_t reserved;      /* must be 0                                       */
  int64_t n_out;         /* N                                               */
  int64_t k_in;          /* K                                               */
  const uint8_t* codes;  /* Q4_0 / NF4 / MXFP4: u8 [N, K/2]; FP8 / Q8_0:
                            u8 [N, K]                                        */
  const void* scales;    /* Q4_0 / Q8_0: fp16 [N, K/32]; NF4: fp32 [N, K/64];
                            FP8: fp32 [1]; MXFP4: u8 (E8M0) [N, K/32];
                            NVFP4: fp32 g, 12 zero bytes, u8 (E4M3)
                            [N, K/16]                                        */
} ql_qweight;

/* ---------------------------------------------------------------- misc */

/* Message for the last failing call on this thread ("" if none). */
const char* ql_last_error(void);

/* Library ABI version (increments on any signature change). */
int32_t ql_version(void);

/* The library's NF4 levels (16 fp32, ascending, c[0] = -1, c[7] = 0,
 * c[15] = 1), built on the host at load time from the normal-quantile
 * construction.  out: host, 16 floats.  Needs no GPU. */
int ql_nf4_levels(float* out);

/* Bytes of scratch that op needs for these shapes (format, N, K, M, r).
 * op = QL_OP_PACK ignores m and r.  Needs no GPU. */
size_t qlora_workspace_bytes(int32_t op, int32_t format, int64_t n_out,
                             int64_t k_in, int64_t m, int32_t r);

/* ---------------------------------------------------------------- a0: pack
 * (Surogate README page, "LoRA & QLoRA" row of the capability table: the base
 * is quantized on load to FP8 or NF4; GGUF-recipe page, "How it works": the
 * base stays in its compressed block form while training.)
 * Quantize fp32 W (dev [N, K]) into codes and scales (dev, layouts above).
 * Once per weight, not per step.  Blocks until the packed data is written
 * (so that non-finite input can be reported): returns QL_ENONFINITE if W
 * holds NaN or Inf (codes and scales are then unspecified), QL_EOVERFLOW if
 * a Q4_0 or Q8_0 scale would exceed the fp16 range.  ws: dev scratch of at least
 * qlora_workspace_bytes(QL_OP_PACK, ...) bytes. */
int quant_pack(int32_t format, const float* w, int64_t n_out, int64_t k_in,
               uint8_t* codes, void* scales, void* ws, size_t ws_bytes,
               void* stream);

/* Dequantize (for verification): out_f32 dev [N, K] gets the exact fp32
 * values, out_bf16 dev [N, K] the one-rounding bf16 values the GEMMs feed to
 * the matrix cores.  Either output may be NULL. */
int qlora_dequant(const ql_qweight* w, float* out_f32, uint16_t* out_bf16,
                  void* stream);

/* ---------------------------------------------------------------- a1: FP8 activations
 * Per-row two-term E4M3 split used by the FP8 base (the pages quantize
 * activations for their FP8 recipe without saying how; this is the reading):
 *   s_m = 2^e, e the smallest integer with 448 * 2^e >= max|x_m|,
 *   t = x / s_m (exact), hi = E4M3(t), lo = E4M3((t - hi) * 16) (the
 *   difference and the factor are exact),  x ~= s_m (hi + lo / 16);
 *   E4M3 = OCP E4M3FN, nearest even.  A zero row gives s_m = 0, codes 0.
 * x: dev bf16 [M, K]; hi, lo: dev u8 [M, K]; scale: dev fp32 [M]. */
int ql_act_quant_e4m3(const uint16_t* x, int64_t m, int64_t k, uint8_t* hi,
                      uint8_t* lo, float* scale, void* stream);

/* ---------------------------------------------------------------- a2-a4: forward
 * y (dev bf16 [M, N]) = x . deq(W)^T + s . U . B^T,  U = x . A^T saved to
 * u_save (dev fp32 [M, r], required).  x: dev bf16 [M, K]; lora_a: dev bf16
 * [r, K]; lora_b: dev bf16 [N, r]; s = alpha / r.  Accumulation is fp32.
 * ws: dev scratch (16-byte aligned), at least qlora_workspace_bytes(
 * QL_OP_FWD, ...) bytes: zero for M > 64; for M <= 64 the contraction is
 * split across workgroups and the fp32 partial sums live there (they are
 * added in a fixed order, so results do not depend on scheduling). */
int qlora_linear_fwd(const ql_qweight* w, const uint16_t* x, int64_t m,
                     const uint16_t* lora_a, const uint16_t* lora_b, int32_t r,
                     float alpha, uint16_t* y, float* u_save, void* ws,
                     size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- a5-a9: backward
 * Given dY (dev bf16 [M, N]), x and the forward's u_save:
 *   dx  (dev bf16 [M, K], may be NULL to skip) = dY . deq(W) + s . V . A,
 *   d_a (dev fp32 [r, K]) = s . V^T . x,   d_b (dev fp32 [N, r]) = s . dY^T . U,
 * with V = dY . B.  accumulate = 0 overwrites d_a / d_b, 1 adds into them.
 * The reductions over M use a fixed split and a fixed summation order.
 * ws: dev scratch, at least qlora_workspace_bytes(QL_OP_BWD, ...) bytes. */
int qlora_linear_bwd(const ql_qweight* w, const uint16_t* x, const uint16_t* dy,
                     const float* u_save, int64_t m, const uint16_t* lora_a,
                     const uint16_t* lora_b, int32_t r, float alpha,
                     uint16_t* dx, float* d_a, float* d_b, int32_t accumulate,
                     void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- backward without a workspace
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * as qlora_linear_bwd (same kernels and launch configuration, so bitwise the
 * same results) except that the scratch is a fixed array inside the library,
 * QL_NOALLOC_SCRATCH_BYTES per GPU, held from module load until the process
 * ends, instead of ws / ws_bytes.  The call allocates nothing.
 * QL_EUNSUPPORTED (nothing enqueued) if the shape needs more scratch than
 * that, i.e. qlora_workspace_bytes(QL_OP_BWD, ...) > QL_NOALLOC_SCRATCH_BYTES:
 * every 4-bit base up to 8192 tokens at Llama-3.1-8B widths fits, the FP8
 * base above about 2000 tokens at Qwen3-8B widths does not.  Every call on one
 * GPU uses that GPU's one array: calls that overlap in time on one GPU (other
 * streams, other host threads) race on it and must be ordered by the caller.
 * Other arguments and errors as qlora_linear_bwd. */
#define QL_NOALLOC_SCRATCH_BYTES (64 * 1024 * 1024)

int qlora_linear_bwd_noalloc(const ql_qweight* w, const uint16_t* x,
                             const uint16_t* dy, const float* u_save, int64_t m,
                             const uint16_t* lora_a, const uint16_t* lora_b,
                             int32_t r, float alpha, uint16_t* dx, float* d_a,
                             float* d_b, int32_t accumulate, void* stream);

/* ---------------------------------------------------------------- groups of independent calls
 * Several independent forward (or backward) calls that share the base
 * format, the token count m and the rank r, in one call: equivalent to
 * calling qlora_linear_fwd (qlora_linear_bwd) for each in order, with bitwise
 * the same results.  At most 64 tokens (the split-contraction path) the
 * group's base GEMMs run as one split launch and one reduction launch instead
 * of two launches per call; the backward's adapter gradients of the whole
 * group take one launch (plus one reduction above 512 tokens) at any token
 * count; other base GEMMs are launched one by one.  In
 * a decoder layer the q, k and v projections (and gate and up) read the same
 * input and form such a group.
 *
 * calls: host array of n (1 .. QL_GROUP_MAX) descriptors with the arguments
 * of the single calls (pointers and ownership as there).  Every call is
 * validated as its single call would be (same error codes); in addition all
 * must use one base format (QL_EINVAL otherwise), and no buffer a call writes
 * (y, u_save, ws; dx, d_a, d_b, ws) may overlap any buffer of another call of
 * the group (QL_EINVAL). */
#define QL_GROUP_MAX 8

typedef struct ql_fwd_call {
  const ql_qweight* w;     /* host pointer to the weight descriptor         */
  const uint16_t* x;       /* dev bf16 [m, K]                                */
  const uint16_t* lora_a;  /* dev bf16 [r, K]                                */
  const uint16_t* lora_b;  /* dev bf16 [N, r]                                */
  float alpha;
  int32_t reserved;        /* must be 0                                      */
  uint16_t* y;             /* dev bf16 [m, N]                                */
  float* u_save;           /* dev fp32 [m, r]                                */
  void* ws;                /* dev scratch, qlora_workspace_bytes(QL_OP_FWD)  */
  size_t ws_bytes;
} ql_fwd_call;

typedef struct ql_bwd_call {
  const ql_qweight* w;
  const uint16_t* x;       /* dev bf16 [m, K]                                */
  const uint16_t* dy;      /* dev bf16 [m, N]                                */
  const float* u_save;     /* dev fp32 [m, r]                                */
  const uint16_t* lora_a;
  const uint16_t* lora_b;
  float alpha;
  int32_t accumulate;      /* 0 overwrite d_a / d_b, 1 add into them         */
  uint16_t* dx;            /* dev bf16 [m, K] or NULL                        */
  float* d_a;              /* dev fp32 [r, K]                                */
  float* d_b;              /* dev fp32 [N, r]                                */
  void* ws;                /* dev scratch, qlora_workspace_bytes(QL_OP_BWD)  */
  size_t ws_bytes;
} ql_bwd_call;

int qlora_linear_fwd_group(const ql_fwd_call* calls, int32_t n, int64_t m,
                           int32_t r, void* stream);
int qlora_linear_bwd_group(const ql_bwd_call* calls, int32_t n, int64_t m,
                           int32_t r, void* stream);

/* ---------------------------------------------------------------- launch plans
 * A plan records a fixed sequence of forward and backward calls (and event
 * markers) once; ql_plan_run then enqueues the whole sequence on a stream in
 * one call; arguments are validated when recorded, so a run does little host
 * work beyond the kernel launches (and a buffer-overlap test while gradient
 * reductions are held back, see below).  With few
 * tokens a layer call's kernels take a few microseconds, less than the host
 * needs to marshal a call from an interpreter, so a step issued call by call
 * leaves the GPU idle between launches; a plan keeps it fed.  (The Soup page's
 * one-layer-at-a-time schedule and the Surogate README's "native kernel
 * dispatch" describe the same need: the host must stay ahead of the GPU.)
 *
 * ql_plan_add_fwd / ql_plan_add_bwd take the arguments of qlora_linear_fwd /
 * qlora_linear_bwd without the stream, validate them exactly as those calls
 * do (same error codes; nothing is recorded on error) and record the call;
 * the ql_qweight is copied, every buffer is referenced, so buffers must stay
 * valid and unchanged in size while the plan is used.  ql_plan_add_event
 * records a marker: at that point of each run, hipEventRecord(event, stream)
 * (event: a hipEvent_t owned by the caller).  ql_plan_run enqueues every
 * recorded step in order on `stream`, with the same kernels and launch
 * configuration as the direct calls, so results are bitwise the same; the
 * one difference is when the dA/dB reductions of backward steps are
 * enqueued: they are gathered into one launch, issued before any later step
 * that touches their outputs or overwrites their workspaces, before every
 * event marker and at the end of the run.  Every output is therefore
 * complete at the plan's end and at each of its events, as with direct
 * calls.  A plan is host data only (no device memory); one plan serves one
 * host thread. */
typedef struct ql_plan ql_plan;

int ql_plan_create(ql_plan** plan);
int ql_plan_add_fwd(ql_plan* plan, const ql_qweight* w, const uint16_t* x,
                    int64_t m, const uint16_t* lora_a, const uint16_t* lora_b,
                    int32_t r, float alpha, uint16_t* y, float* u_save, void* ws,
                    size_t ws_bytes);
int ql_plan_add_bwd(ql_plan* plan, const ql_qweight* w, const uint16_t* x,
                    const uint16_t* dy, const float* u_save, int64_t m,
                    const uint16_t* lora_a, const uint16_t* lora_b, int32_t r,
                    float alpha, uint16_t* dx, float* d_a, float* d_b,
                    int32_t accumulate, void* ws, size_t ws_bytes);
/* a group of independent calls (as qlora_linear_fwd_group / _bwd_group) */
int ql_plan_add_fwd_group(ql_plan* plan, const ql_fwd_call* calls, int32_t n,
                          int64_t m, int32_t r);
int ql_plan_add_bwd_group(ql_plan* plan, const ql_bwd_call* calls, int32_t n,
                          int64_t m, int32_t r);
int ql_plan_add_event(ql_plan* plan, void* event);
/* number of recorded steps (0 for NULL) */
int ql_plan_size(const ql_plan* plan);
int ql_plan_run(ql_plan* plan, void* stream);
int ql_plan_destroy(ql_plan* plan);

/* ---------------------------------------------------------------- stacked adapters
 * Frozen lower adapters under one trainable top adapter (the Surogate review
 * page's stacked LoRA: adapters trained on top of other adapters with no
 * offline merge; the README's "LoRA & QLoRA" row).  With adapter i = (A_i
 * [r_i, K], B_i [N, r_i], s_i = alpha_i / r_i), the top one last,
 *   y = x.W^T + sum_i s_i.(x.A_i^T).B_i^T  equals one adapter of rank
 *   R = sum_i r_i:  A = [A_1; ...; A_top],  B = [c_1 B_1, ..., B_top],
 *   c_i = s_i / s_top, scale s_top (alpha_cat = s_top * R),
 * and so does dX; the top adapter's gradients are rows [R - r_top, R) of dA
 * and columns [R - r_top, R) of dB of the backward call with (A, B, R,
 * alpha_cat).  ql_stack_adapters writes A (a_cat, dev bf16 [R, K]) and B
 * (b_cat, dev bf16 [N, R]) once per change of the adapters: A's rows and the
 * top block of B are copied, each frozen block of B is bf16(fl32(c_i) * B_i)
 * (exact when c_i is a power of two).  *alpha_cat (host) receives alpha_cat.
 * adapters: host array of n (2 .. QL_STACK_MAX) descriptors, device
 * pointers 16-byte aligned.  QL_EUNSUPPORTED if R is not 8, 16 or 32;
 * QL_EINVAL for a null or misaligned pointer, r_i < 1, alpha_i not finite
 * and positive. */
#define QL_STACK_MAX 8

typedef struct ql_adapter {
  const uint16_t* lora_a;  /* dev bf16 [r, K]                               */
  const uint16_t* lora_b;  /* dev bf16 [N, r]                               */
  int32_t r;
  float alpha;
} ql_adapter;

int ql_stack_adapters(const ql_adapter* adapters, int32_t n, int64_t n_out,
                      int64_t k_in, uint16_t* a_cat, uint16_t* b_cat,
                      float* alpha_cat, void* stream);

/* ---------------------------------------------------------------- adapter optimizer step
 * One AdamW step on the adapters, every listed tensor in one launch.  The
 * Surogate README page lists "AdamW 8-bit" among its optimizers and the
 * GGUF-recipe page ("How it works") trains the adapters with 8-bit AdamW; the
 * update is decoupled weight decay (Loshchilov & Hutter, "Decoupled Weight
 * Decay Regularization", Algorithm 2) in the PyTorch / bitsandbytes
 * convention (decay scaled by the learning rate, applied first).  Per
 * element, g = grad * grad_scale, t = step (>= 1, counting this update):
 *   param      *= 1 - lr * weight_decay
 *   exp_avg     = beta1 * exp_avg + (1 - beta1) * g
 *   exp_avg_sq  = beta2 * exp_avg_sq + (1 - beta2) * g^2
 *   param      -= lr / (1 - beta1^t) * exp_avg
 *                 / (sqrt(exp_avg_sq) / sqrt(1 - beta2^t) + eps)
 *   param_bf16  = bf16(param), nearest even (skipped when NULL)
 * in fp32; the per-step constants (1 - lr * weight_decay, 1 - beta,
 * lr / (1 - beta1^t), 1 / sqrt(1 - beta2^t)) are formed in fp64 on the host
 * and rounded once.  The
 * moments are fp32: the 8-bit state format of the pages' optimizer is not
 * defined there.  param, exp_avg and exp_avg_sq are updated in place; grad is
 * only read (d_a / d_b of qlora_linear_bwd, fp32).
 *
 * tensors: host array of n_tensors (0 .. QL_ADAMW_MAX_TENSORS) descriptors;
 * every pointer dev, 16-byte aligned, n a multiple of 4 (n = 0 is skipped);
 * the arrays of one tensor must not overlap each other or another tensor's.
 * hp: host.  Errors (QL_EINVAL): bad count, pointer or size; step < 1;
 * beta outside [0, 1); negative lr, eps or weight_decay; non-finite values. */
#define QL_ADAMW_MAX_TENSORS 32

typedef struct ql_adamw_tensor {
  float* param;          /* dev fp32 [n], master adapter weights            */
  const float* grad;     /* dev fp32 [n]                                    */
  float* exp_avg;        /* dev fp32 [n], first moment                      */
  float* exp_avg_sq;     /* dev fp32 [n], second moment                     */
  uint16_t* param_bf16;  /* dev bf16 [n] or NULL: copy for the layer        */
  int64_t n;             /* elements                                        */
} ql_adamw_tensor;

typedef struct ql_adamw_hparams {
  /* fp64, so that 1 - beta2 and the bias corrections are formed from the
     caller's exact values before the one rounding to fp32 */
  double lr, beta1, beta2, eps, weight_decay, grad_scale;
  int32_t step;          /* t >= 1 */
  int32_t reserved;      /* must be 0 */
} ql_adamw_hparams;

int ql_adamw_step(const ql_adamw_tensor* tensors, int32_t n_tensors,
                  const ql_adamw_hparams* hp, void* stream);

/* ---------------------------------------------------------------- adapter optimizer step, 8-bit state
 * The same AdamW step with 8-bit moments, the state format of the pages' 8-bit
 * AdamW (Surogate README page, "Optimizers & monitoring" row; GGUF-recipe page,
 * "How it works") taken from Dettmers et al., "8-bit Optimizers via Block-wise
 * Quantization": each moment is stored as one code per element plus one fp32
 * scale (the block's largest magnitude) per QL_ADAMW8_BLOCK consecutive
 * elements; a code stands for level * scale, level from the dynamic tree type:
 * magnitude bits = z zero bits, a one bit, f bits holding q, level
 * 10^-z * (0.1 + 0.9 (q + 1) / 2^f), all-zero bits 0 (ql_dyn8_levels).  The
 * first moment uses the signed type (bit 7 the sign, 7 magnitude bits), the
 * second the unsigned one (8 magnitude bits).  Per element: dequantize, the
 * update of ql_adamw_step in fp32 (the parameter moves with the fp32 moments),
 * then per block: scale = largest |new moment|, code = number of decision
 * thresholds fl32(fl32(l_i + l_i+1) * 0.5) below |m / scale| (IEEE divide; a
 * value on a threshold takes the lower code), sign bit for a negative first
 * moment with a non-zero code; a block whose scale is 0 stores codes 0.
 * Every fp32 operation rounds once, in a fixed order, so results are
 * reproducible bit for bit.  A zero state (codes 0, scales 0) is the start.
 *
 * tensors: host array of n_tensors (0 .. QL_ADAMW_MAX_TENSORS) descriptors;
 * n a multiple of 8 (0 skips the tensor); param, grad, param_bf16 dev and
 * 16-byte aligned, codes dev and 8-byte aligned, scales dev fp32
 * [ceil(n / QL_ADAMW8_BLOCK)].  hp and errors as ql_adamw_step. */
#define QL_ADAMW8_BLOCK 2048

typedef struct ql_adamw8_tensor {
  float* param;              /* dev fp32 [n], master adapter weights        */
  const float* grad;         /* dev fp32 [n]                                */
  uint8_t* exp_avg;          /* dev u8 [n], first-moment codes (signed)     */
  float* exp_avg_absmax;     /* dev fp32 [ceil(n / QL_ADAMW8_BLOCK)]        */
  uint8_t* exp_avg_sq;       /* dev u8 [n], second-moment codes (unsigned)  */
  float* exp_avg_sq_absmax;  /* dev fp32 [ceil(n / QL_ADAMW8_BLOCK)]        */
  uint16_t* param_bf16;      /* dev bf16 [n] or NULL: copy for the layer    */
  int64_t n;                 /* elements                                    */
} ql_adamw8_tensor;

int ql_adamw8_step(const ql_adamw8_tensor* tensors, int32_t n_tensors,
                   const ql_adamw_hparams* hp, void* stream);

/* The levels of the 8-bit state type, indexed by the magnitude bits
 * (ascending): is_signed != 0 gives the 128 magnitudes of the signed type,
 * 0 the 256 levels of the unsigned one.  out: host floats.  Needs no GPU. */
int ql_dyn8_levels(int32_t is_signed, float* out);

/* ---------------------------------------------------------------- a10: layer stream
 * (Soup page, opening paragraph.)  The frozen base is kept in page-locked
 * host memory; a few device slots, allocated once by the caller, each hold
 * one decoder layer's packed weights, and the copy of the next layer runs on
 * a side stream while the current one computes.
 *
 * The caller allocates n_slots device buffers of slot_bytes each (slot_dev,
 * 256-byte aligned) and n_layers pinned host images (layer_host, page-locked,
 * layer_bytes[l] <= slot_bytes).  The pool owns only HIP events and
 * bookkeeping; it never allocates device or host memory.  One pool serves
 * one host thread.
 *
 * layer_stream_prefetch: make layer l resident in some slot.  A hit (l
 *   already resident or in flight) enqueues nothing.  A miss picks an empty
 *   slot, else the least recently released one, makes copy_stream wait until
 *   the compute stream has released that slot, then enqueues the
 *   host-to-device copy on copy_stream and records the slot's ready event.
 *   QL_ESTATE if every slot holds a layer that is prefetched or acquired but
 *   not yet released.
 * ql_pool_acquire: compute_stream waits for layer l's ready event; *slot_dev
 *   receives the slot's device address.  QL_ESTATE if l was not prefetched
 *   or is already acquired.
 * ql_pool_release: records on compute_stream that the slot's readers are
 *   enqueued, so a later copy into it waits for them.  QL_ESTATE if l is not
 *   acquired. */
typedef struct ql_pool ql_pool;

int ql_pool_create(ql_pool** pool, int32_t n_slots, void* const* slot_dev,
                   size_t slot_bytes, int32_t n_layers,
                   const void* const* layer_host, const size_t* layer_bytes);
int layer_stream_prefetch(ql_pool* pool, int32_t layer, void* copy_stream);
int ql_pool_acquire(ql_pool* pool, int32_t layer, void* compute_stream,
                    void** slot_dev);
int ql_pool_release(ql_pool* pool, int32_t layer, void* compute_stream);
/* counters: out[0] prefetch hits, out[1] copies issued, out[2] bytes copied */
int ql_pool_stats(const ql_pool* pool, int64_t* out3);
/* Test hooks, host-forced conditions only: delay_us > 0 makes each copy wait
 * that long on the copy stream before it starts (a host function on the
 * stream); poison != 0 fills a slot with 0xFF bytes before each copy (every
 * bf16/fp32 read of it is NaN); skip_wait != 0 makes acquire skip the
 * compute-stream wait (a deliberate race, for a negative control only). */
int ql_pool_debug(ql_pool* pool, int32_t delay_us, int32_t poison,
                  int32_t skip_wait);
/* Blocks until every copy the pool has enqueued has finished, then frees the
 * pool's events and bookkeeping (the caller's slots and images are not
 * touched).  QL_EHIP if waiting for a copy failed; the pool is freed anyway. */
int ql_pool_destroy(ql_pool* pool);

/* ---------------------------------------------------------------- measurement
 * The HBM ceiling the kernels are measured against: one pass of a plain
 * streaming read over buf (dev, 16-byte aligned, bytes a positive multiple of
 * 16), every 16-byte word read once by a grid of QL_STREAM_READ_THREADS
 * threads (256 workgroups of 256, eight loads in flight per thread, strided
 * by the grid), each thread's words folded by XOR into sink[thread] (dev
 * uint32 [QL_STREAM_READ_THREADS]), so the XOR of all of sink is the XOR of
 * every 32-bit word of buf.  Asynchronous on stream.  QL_EINVAL for a null
 * or misaligned pointer or a bad size. */
#define QL_STREAM_READ_THREADS 65536
int ql_stream_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_H */
