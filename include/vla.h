/*
 * vla.h -- C ABI of the dual-phase policy step on AMD Instinct MI355X (gfx950).
 *
 * A bidirectional prefix pass encodes an observation once and writes an explicit
 * cross-attention K/V cache; a flow-matching action expert then refines a noise
 * chunk over T Euler steps, reading that cache at every step.
 *
 * Sources ("the paper" is vla.cpp: A Unified Inference Runtime for
 * Vision-Language-Action Models, arXiv 2606.08094; "the reading notes" are the
 * paper.gecl.asia notes on it):
 *   - prefix computed once per observation, its projections reused by every
 *     solver step, refreshed on each new observation; graphs and buffers kept
 *     for unchanged shapes ............................... the paper, §III-B
 *   - cross-attention K_C = Z W_K, V_C = Z W_V, softmax(Q K_C^T/sqrt(d_k) + M) V_C,
 *     M = -inf on padded prefix keys, 0 elsewhere ........ the paper, §III-B, Eq. 2
 *   - joint attention: each prefix layer's own keys and values are the cache,
 *     and the action tokens' keys and values are appended to them in one
 *     softmax (the pi0 form) ............................. the paper, §III-B
 *   - Euler solver X^{k+1} = X^k + (tau_{k+1} - tau_k) v(X^k, tau_k)
 *                                                          the paper, §III-A, Eq. 1
 *   - bidirectional prefix mask; hidden states taken before the LM output
 *     projection ........................................ the reading notes, Method 1-2
 *   - ternary W2A8 linear ............................... the paper, §III-D, Eq. 4
 *   - a request returns the chunk and its dimensions, "or an error"
 *                                                          the paper, §III-C
 *
 * Conventions for every entry point:
 *   - Device pointers are HIP device addresses on the current device; "host"
 *     pointers are ordinary CPU memory.  `stream` is a hipStream_t (NULL = the
 *     null stream).  Work is enqueued asynchronously on `stream`; the returned
 *     status covers argument/shape validation and launch errors, and a device
 *     fault surfaces at the caller's next synchronising call.
 *   - On any status other than VLA_OK no output buffer has been written.
 *   - The library never aborts or exits; vla_last_error() gives a per-thread
 *     message for the last failing call.
 *   - Calls on one model come from one host thread at a time.  On the device,
 *     a prefix encode and a denoise of the same model may run concurrently on
 *     different streams (they use separate parts of the model's workspace) if
 *     they use different cache storage and neither asks for timings; two
 *     encodes, or two denoises, of one model must not overlap.  A call that
 *     has to grow the workspace (a larger batch or prefix than before)
 *     synchronises the device first.  Different models are independent.
 */
#ifndef VLA_H_
#define VLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VLA_ABI_VERSION 2

typedef enum {
  VLA_OK = 0,
  VLA_ERR_INVALID_ARGUMENT = 1, /* null pointer, non-positive size, bad value   */
  VLA_ERR_SHAPE_MISMATCH = 2,   /* sizes disagree with the model or the cache   */
  VLA_ERR_INVALID_HANDLE = 3,   /* released, foreign or corrupted handle        */
  VLA_ERR_UNSUPPORTED = 4,      /* a shape or mode the library does not support */
  VLA_ERR_OUT_OF_MEMORY = 5,    /* a device allocation failed                   */
  VLA_ERR_DEVICE = 6            /* no usable gfx950 device, or a HIP call failed */
} vla_status;

typedef enum {
  VLA_F32 = 0,       /* every weight and activation float32                       */
  VLA_BF16 = 1,      /* bf16 weights and GEMM operands, fp32 residual and softmax  */
  VLA_W2A8_BF16 = 2  /* prefix linears ternary W2A8 (Eq. 4), the rest as VLA_BF16  */
} vla_precision;

typedef enum { VLA_OUT_F32 = 0, VLA_OUT_BF16 = 1 } vla_out_dtype;

/* Element type of the prefix hidden states handed to vla_prefix_encode_ex. */
typedef enum { VLA_IN_F32 = 0, VLA_IN_BF16 = 1 } vla_in_dtype;

/* How the action expert reads the observation (the paper, §III-B).
 * CROSS: the final prefix states Z are projected into per-expert-layer K_C, V_C
 *   (Eq. 2), and every expert layer has self-attention over the chunk, then
 *   cross-attention into its K_C, V_C, then the MLP.
 * JOINT: the cache holds every prefix layer's own keys and values; expert layer
 *   l attends, in one softmax, over prefix layer l's keys followed by the
 *   chunk's own keys (prefix tokens never see the chunk: their keys and values
 *   come from the prefix pass alone), then runs the MLP.  Needs L_e == L_p,
 *   Hkv_e == Hkv, hd_e == hd and precision VLA_F32 or VLA_BF16. */
typedef enum { VLA_ATTN_CROSS = 0, VLA_ATTN_JOINT = 1 } vla_attn_mode;

/* Model shape.  Prefix: d_p wide, L_p layers, Hq query heads sharing Hkv
 * key/value heads of width hd, GeGLU width F_p.  Expert: the same fields with
 * suffix _e.  H x d_a is the action chunk (d_a <= 256).  Requirements:
 * Hq % Hkv == 0 and Hq_e % Hkv_e == 0; for VLA_F32, hd and hd_e in {32, 64}
 * and d_p, d_e, F_p, F_e multiples of 16; otherwise hd and hd_e in
 * {64, 128, 256}, d_p, d_e, F_p, F_e multiples of 64 and d_e <= 4096, and for
 * VLA_W2A8_BF16 also d_p, F_p and Hq*hd multiples of 128. */
typedef struct {
  int32_t abi_version; /* must be VLA_ABI_VERSION */
  int32_t precision;   /* vla_precision */
  int32_t d_p, L_p, Hq, Hkv, hd, F_p;
  int32_t d_e, L_e, Hq_e, Hkv_e, hd_e, F_e;
  int32_t H, d_a;
  float rms_eps;       /* RMSNorm epsilon, e.g. 1e-6 */
  int32_t attn_mode;   /* vla_attn_mode */
} vla_model_config;

/* Weights, all linear layers [out, in] row-major (y = x W^T), in this order:
 *   per prefix layer l = 0..L_p-1:  w1[d_p] wq[Hq*hd, d_p] wk[Hkv*hd, d_p]
 *       wv[Hkv*hd, d_p] wo[d_p, Hq*hd] w2[d_p] wg[F_p, d_p] wu[F_p, d_p] wd[d_p, F_p]
 *   prefix final norm gain [d_p]
 *   per expert layer e: cache wk[Hkv_e*hd_e, d_p], cache wv[Hkv_e*hd_e, d_p]
 *   w_in[d_e, d_a]
 *   per expert layer e:  a1[d_e] wqs[Hq_e*hd_e, d_e] wks[Hkv_e*hd_e, d_e]
 *       wvs[Hkv_e*hd_e, d_e] wos[d_e, Hq_e*hd_e] a2[d_e] wqc[Hq_e*hd_e, d_e]
 *       woc[d_e, Hq_e*hd_e] a3[d_e] wg[F_e, d_e] wu[F_e, d_e] wd[d_e, F_e]
 *   expert final norm gain [d_e], w_out[d_a, d_e]
 * With VLA_ATTN_JOINT there is no prefix final norm, no cache projection and
 * no cross-attention: the prefix layers as above, then w_in, then per expert
 * layer a1 wqs wks wvs wos a3 wg wu wd, then the expert final norm and w_out.
 * RMSNorm gains ("w1", "a1", final norms ...) are float32 and applied as (1 + w).
 * Linear weights are float32 for VLA_F32 and bfloat16 otherwise, except that
 * with VLA_W2A8_BF16 the seven prefix linears of every layer (wq wk wv
 * wo wg wu wd) are packed ternary: uint8 [out, in/4], four 2-bit codes per byte,
 * code = q + 1, element 4j+i of a row in bits 2i..2i+1 of byte j (code 3 is
 * invalid); their fp32 scales beta are listed, in the same order, in
 * `ternary_beta` (host memory, 7 * L_p entries).
 * The library copies every weight into its own layout during vla_model_create;
 * the caller's buffers may be freed once it returns. */
typedef struct {
  const void* const* tensors; /* host array of n_tensors pointers: device or host memory */
  int32_t n_tensors;          /* must equal vla_n_tensors(cfg)            */
  const float* ternary_beta;  /* host; NULL unless precision is W2A8      */
} vla_weights;

/* Integration schedule of Eq. 1.  If `schedule` is non-NULL it is a host array
 * of steps + 1 times tau_0..tau_T; otherwise tau_k = tau_start + k (tau_end -
 * tau_start) / steps.  Passing NULL for the whole struct means 0 -> 1. */
typedef struct {
  float tau_start, tau_end;
  const float* schedule;
} vla_solver;

/* Optional per-call timings (filled only when a pointer is passed; that makes
 * the call synchronise its stream). */
typedef struct {
  float prefix_ms;        /* vla_prefix_encode: whole call on the device      */
  float denoise_ms;       /* vla_denoise_chunk: all steps on the device       */
  float step_ms;          /* denoise_ms / steps                               */
  int32_t graph_replayed; /* 1 if the solver loop replayed a cached HIP graph */
} vla_timing;

typedef struct vla_model vla_model;
typedef struct vla_kv_cache vla_kv_cache;

/* Human-readable name of a status, and the calling thread's last error message. */
const char* vla_status_string(vla_status s);
const char* vla_last_error(void);

/* Number of weight tensors the model config expects (-1 if cfg is invalid). */
int32_t vla_n_tensors(const vla_model_config* cfg);

/* Shape and kind of tensor `index` in the order above: rows x cols (cols = 1 for
 * gains); kind 0 = fp32 gain, 1 = linear (fp32 or bf16 by precision), 2 = packed
 * ternary (cols is the packed byte count in/4). */
vla_status vla_tensor_info(const vla_model_config* cfg, int32_t index, int64_t* rows,
                           int64_t* cols, int32_t* kind);

/* Build a model on the current device: validates cfg, copies and repacks the
 * weights (ternary codes are checked; an invalid code 3 gives
 * VLA_ERR_INVALID_ARGUMENT), and owns the result until vla_model_destroy; the
 * caller's tensors are only read during the call.  A tensor may be in device
 * memory or in host memory (pageable or pinned, each read once through the
 * library's staging buffer): with every tensor on the host the device holds
 * the packed model plus one staging buffer, never a second copy of the
 * weights.  Synchronises `stream`.  Returns VLA_ERR_DEVICE if no gfx950
 * device is present. */
vla_status vla_model_create(const vla_model_config* cfg, const vla_weights* weights,
                            void* stream, vla_model** out);
vla_status vla_model_destroy(vla_model* model);

/* Bytes of K/V cache storage for `batch` observations of `n_prefix` tokens:
 * blocks [batch][L_e][2 (K, V)][Hkv_e], each of Np x hd_e elements (with
 * VLA_ATTN_JOINT, block l holds prefix layer l's keys and values), then, at
 * the next multiple of 256 bytes, `batch` int32 prefix lengths (written by
 * vla_prefix_encode_masked), the total rounded up to a multiple of 256.
 * VLA_F32: float32, Np = n_prefix, element (t, d) at t * hd_e + d.
 * Otherwise bfloat16 in the operand orders of the 16x16x32 MFMA, Np = n_prefix
 * rounded up to a multiple of 32 (padding rows hold zero):
 *   K block: (t, d) at ((((t/16) * (hd_e/32) + d/32) * 64 + t%16 + 16*((d/8)%4)) * 8 + d%8
 *   V block: with u = t%32, (t, d) at
 *            ((((t/32) * (hd_e/16) + d/16) * 64 + d%16 + 16*((u%16)/4)) * 8 + 4*(u/16) + u%4
 * For one observation of a bf16 cross-attention model whose solver runs the
 * absorbed cross sublayer (chunk of 17 to 64 rows, expert width a multiple
 * of 128 up to 1024, Hq_e <= 32, Np <= 512 and Hq_e * Np <= 4096, unless the
 * model was created with VLA_ABSORB=0 in the environment), the lengths are
 * followed by per-layer products of the cached keys and values that the
 * encode also writes and the denoise reads instead of them (the same
 * attention, other rounding points): Wq_j^T K^T and V Wo_j^T for every query
 * head j, 2 * L_e * Hq_e * Np * d_e bf16 elements, and the values once more,
 * L_e * Hkv_e * Np * hd_e elements; their layout is internal.
 * Returns 0 for invalid arguments. */
size_t vla_kv_cache_bytes(const vla_model* model, int32_t batch, int32_t n_prefix);

/* Prefix pass (the paper, §III-B; the reading notes, Method 1-3): encodes
 * `batch` observations of `n_prefix` tokens, prefix_hidden = device float32
 * [batch][n_prefix][d_p], through L_p bidirectional layers and the final
 * RMSNorm, and projects the result into every expert layer's K and V, written
 * to `kv_storage` (device, caller-owned, >= vla_kv_cache_bytes bytes, layout as
 * above).  With VLA_ATTN_JOINT each layer's keys and values go to the cache
 * instead (the last layer stops after its keys and values: nothing reads the
 * rest).  *out receives a handle that refers to kv_storage; it stays valid
 * until vla_kv_cache_release and may serve any number of denoise calls.
 * `timing` (nullable) receives prefix_ms and makes the call synchronise. */
vla_status vla_prefix_encode(vla_model* model, const float* prefix_hidden, int32_t batch,
                             int32_t n_prefix, void* kv_storage, size_t kv_bytes,
                             void* stream, vla_kv_cache** out, vla_timing* timing);

/* vla_prefix_encode for observations of different lengths (key padding, the
 * paper §III-B, Eq. 2: M = 0 for visible keys, -inf for masked ones).
 * lengths: host int32 [batch], 1 <= lengths[b] <= n_prefix; observation b fills
 * the first lengths[b] rows of its [n_prefix][d_p] block and the rest is
 * padding, whose content is ignored (the library zeroes it on the way in).
 * Every softmax that reads prefix keys -- the prefix attention, the expert's
 * cross-attention and the prefix part of joint attention -- gives the padded
 * keys weight 0, so an observation's chunk is that of the same observation
 * encoded alone at its length.  lengths == NULL is vla_prefix_encode.  The
 * lengths are kept in the cache storage's tail for the denoise calls.
 * VLA_ERR_INVALID_ARGUMENT for a length outside 1..n_prefix (nothing written). */
vla_status vla_prefix_encode_masked(vla_model* model, const float* prefix_hidden, int32_t batch,
                                    int32_t n_prefix, const int32_t* lengths, void* kv_storage,
                                    size_t kv_bytes, void* stream, vla_kv_cache** out,
                                    vla_timing* timing);

/* vla_prefix_encode_masked with the element type of prefix_hidden given:
 * in_dtype VLA_IN_F32 (device float32, as above) or VLA_IN_BF16 (device
 * bfloat16 [batch][n_prefix][d_p], for callers whose vision and text encoders
 * produce bf16 states; each value is widened exactly to the float32 residual
 * stream, so the result equals vla_prefix_encode_masked on the widened
 * tensor, bit for bit).  Any precision of the model accepts either type.
 * VLA_ERR_INVALID_ARGUMENT for another in_dtype; the rest as
 * vla_prefix_encode_masked (lengths == NULL: no key padding). */
vla_status vla_prefix_encode_ex(vla_model* model, const void* prefix_hidden, int32_t in_dtype,
                                int32_t batch, int32_t n_prefix, const int32_t* lengths,
                                void* kv_storage, size_t kv_bytes, void* stream,
                                vla_kv_cache** out, vla_timing* timing);

/* Flow-matching solver (the paper, §III-A, Eq. 1): X^0 = noise (device float32
 * [batch][H][d_a], batch and n_prefix taken from the cache), `steps` Euler
 * steps of the action expert over the cached K/V, X^T written to actions_out
 * (device [batch][H][d_a], float32 or bfloat16 by out_dtype).  The step loop
 * runs as a HIP graph captured once per (cache storage, prefix lengths, batch,
 * n_prefix, steps) and replayed afterwards; the model keeps the 8 most
 * recently used graphs.  noise and actions_out may alias. */
vla_status vla_denoise_chunk(vla_model* model, const vla_kv_cache* kv, const float* noise,
                             int32_t steps, const vla_solver* solver, void* actions_out,
                             int32_t out_dtype, void* stream, vla_timing* timing);

/* Release a cache handle (the storage stays the caller's). */
vla_status vla_kv_cache_release(vla_kv_cache* kv);

/* Batch and prefix length a cache was encoded with. */
vla_status vla_kv_cache_info(const vla_kv_cache* kv, int32_t* batch, int32_t* n_prefix);

/* The prefix's bf16 product as a unit (the paper, §III-B: every linear of the
 * bidirectional prefix): out = A W^T in float32 accumulation on the same
 * kernels the prefix uses (both operands repacked into the MFMA fragment
 * layout first; more than 64 rows on the 288-row-tile kernels, or for the
 * residual form at up to 320 rows the whole-K row tiles of the prefix's O
 * projection, fewer on the chunk-sized kernel, K splits summed in a fixed
 * order).  a: device bf16 bit patterns [M][K], w: device bf16 [N][K],
 * row-major.  epilogue VLA_GEMM_STORE: out is device float32 [M][N].
 * VLA_GEMM_GEGLU: w's rows are gate and up interleaved in blocks of 16 (rows
 * 32 b .. 32 b + 15 are gate features 16 b .. 16 b + 15, the next 16 rows their
 * up features, as the model's gate/up weight) and out is [M][N / 2] =
 * GELU(gate) * up.  VLA_GEMM_RESIDUAL: out is device float32 [M][N], read and
 * updated in place, out += A W^T (the residual update of the prefix's O
 * projection).  Any other value: VLA_ERR_INVALID_ARGUMENT.  K % 64 == 0,
 * N % 32 == 0.  Allocates staging and synchronises `stream`: for tests, not a
 * hot path. */
#define VLA_GEMM_STORE 0
#define VLA_GEMM_GEGLU 1
#define VLA_GEMM_RESIDUAL 2
vla_status vla_gemm_bf16(const uint16_t* a, const uint16_t* w, int32_t M, int32_t N, int32_t K,
                         int32_t epilogue, float* out, void* stream);

/* Per-row int8 quantization of Eq. 4 (the paper, §III-D): for each row m of
 * x (device float32 [M][K]) alpha[m] = max(max_j |x_mj|, 1e-5) / 127 and
 * a[m][j] = clip(rint(x_mj / alpha[m]), -128, 127), IEEE float32 division,
 * ties to even.  Outputs: a (device int8 [M][K]), alpha (device float32 [M]). */
vla_status vla_quantize_rows_i8(const float* x, int32_t M, int32_t K, int8_t* a,
                                float* alpha, void* stream);

/* Ternary W2A8 GEMM of Eq. 4: acc[m][n] = sum_j a[m][j] q[n][j] in int32, with
 * q unpacked from q_packed (device uint8 [N][K/4], format as above; K % 128 == 0),
 * and y[m][n] = bf16(float(acc) * (alpha[m] * beta)) rounded to nearest even.
 * a: device int8 [M][K]; alpha: device float32 [M]; acc_out (device int32
 * [M][N]) may be NULL; y_bf16 (device uint16 bit patterns [M][N]) may be NULL. */
vla_status vla_w2a8_gemm(const int8_t* a, const float* alpha, const uint8_t* q_packed,
                         float beta, int32_t M, int32_t N, int32_t K, int32_t* acc_out,
                         uint16_t* y_bf16, void* stream);

/* The same GEMM with group-wise weight scales (the paper, §III-D, Eq. 4's
 * beta_g(n)): output channel n is scaled by beta[n / group] (host float32,
 * N / group entries; group must divide N; group == N is the per-tensor form of
 * vla_w2a8_gemm), and `path` picks the kernel: VLA_W2A8_MFMA, the int8
 * matrix-core kernel the model uses (K % 128 == 0, N % 32 == 0), or
 * VLA_W2A8_DOT4, a vector-ALU kernel on v_dot4_i32_i8 (K % 64 == 0), the
 * counterpart of the page's dp4a path kept for comparison.  Both give the same
 * int32 accumulators bit for bit.  kernel_ms (host, nullable) receives the
 * GEMM kernel's device time.  Synchronises `stream`. */
typedef enum { VLA_W2A8_MFMA = 0, VLA_W2A8_DOT4 = 1 } vla_w2a8_path;
vla_status vla_w2a8_gemm_ex(const int8_t* a, const float* alpha, const uint8_t* q_packed,
                            const float* beta, int32_t group, int32_t path, int32_t M, int32_t N,
                            int32_t K, int32_t* acc_out, uint16_t* y_bf16, void* stream,
                            float* kernel_ms);

/* vla_w2a8_gemm for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * same arguments, same results bit for bit, but the repacked weights and the
 * invalid-code flag live in a fixed 16 MiB scratch array that the library
 * holds on each device it runs on until the process ends, so this call makes
 * no hipMalloc, hipFree or other allocating call.  N * K / 4 must not exceed
 * 16 MiB - 256 bytes (VLA_ERR_UNSUPPORTED otherwise).  Every call on a device
 * reuses that device's scratch: calls that overlap on one device (another
 * thread, or another stream before this one has returned) race and give
 * undefined results.  Synchronises `stream`. */
vla_status vla_w2a8_gemm_noalloc(const int8_t* a, const float* alpha, const uint8_t* q_packed,
                                 float beta, int32_t M, int32_t N, int32_t K, int32_t* acc_out,
                                 uint16_t* y_bf16, void* stream);

/* Host helpers for the packed ternary format: pack codes q in {-1, 0, 1}
 * (host int8 [N][K], K % 4 == 0) into host uint8 [N][K/4]; unpack the reverse
 * (VLA_ERR_INVALID_ARGUMENT on a code 3). */
vla_status vla_ternary_pack(const int8_t* q, int32_t N, int32_t K, uint8_t* packed);
vla_status vla_ternary_unpack(const uint8_t* packed, int32_t N, int32_t K, int8_t* q);

/* Kernel probes for measurement (timing one kernel class with HIP events) are
 * declared in vla_probe.h. */

#ifdef __cplusplus
}
#endif
#endif /* VLA_H_ */
