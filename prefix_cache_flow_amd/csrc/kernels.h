// Host-side launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace vla {

// Two byte ranges that extra workgroups of a kernel read once and drop, so that
// a later kernel (which streams them) finds them in cache instead of waiting
// on HBM.  `blocks` workgroups are added to the grid.
// With group > 0 a range is read XCD by XCD: the consuming kernel's workgroup
// for column group g of `group` bytes runs on XCD g % 8 (workgroups go to the
// eight XCDs round robin), so the extra workgroups on XCD c read the groups
// g = c (mod 8) into that XCD's L2, where the consumer finds them.
struct Prefetch {
  const void* p = nullptr;
  size_t bytes = 0, group = 0;
  const void* p2 = nullptr;
  size_t bytes2 = 0, group2 = 0;
  const void* p3 = nullptr;
  size_t bytes3 = 0, group3 = 0;
  unsigned* sink = nullptr;  // 64 words, written only for an impossible value
  int blocks = 0;
};
// Grid depth for a kernel whose own grid layer holds `per` workgroups: whole
// layers of prefetch workgroups after it, at least `blocks` of them.
inline int prefetch_depth(int per, int blocks) { return blocks > 0 ? 1 + (blocks + per - 1) / per : 1; }

// ------------------------------------------------------------------ epilogues
// What a GEMM does with its fp32 result v at (m, n).
enum EpiKind {
  EPI_STORE = 0,  // out[m * ldo + n] = v                       (bf16 or fp32)
  EPI_RESID = 1,  // resid[m * ldr + n] += v                     (fp32 residual)
  EPI_GEGLU = 2,  // gate/up rows interleaved in blocks of 16: column n = 32 b + i is
                  // gate feature 16 b + i for i < 16, up feature 16 b + i - 16 otherwise;
                  // out[m * ldo + f] = GELU(gate_f) * up_f     (bf16 or fp32)
  EPI_CACHE = 3,  // K/V cache scatter: row m = (b, t) with b = m / npre, t = m % npre;
                  // column n = ((l * 2 + kv) * hkv + h) * hd + d; block
                  // ((b * L + l) * 2 + kv) * hkv + h of npad * hd elements holds
                  // (t, d) row-major (out_frag == 0) or, with out_frag, K in
                  // frag_idx and V in vfrag_idx order (common.h)
  EPI_PARTIAL = 4,// raw fp32 partial sums to ws[split][m][n], left for a row kernel
  EPI_QKV = 5,    // fused self-attention projection, row m = (b, t) with b = m / npre:
                  // columns n < nq go to out[m * ldo + n] (rows), the next hkv * hd
                  // to kout and the last hkv * hd to vout, in blocks of npad * hd
                  // elements, block h of batch b at (b * kv_bs / (npad * hd) + h)
                  // (kv_bs = 0: hkv * npad * hd); bf16 K / V in frag_idx /
                  // vfrag_idx order, fp32 (out_f32) as rows t * hd + d
  EPI_SCORES = 6  // cross-attention scores in log2 units, one observation: column
                  // n = j * npad + t is key t of query head j (npad keys per head, a
                  // multiple of 32); keys t >= klen[0] (or npre when klen is null)
                  // are masked.  Per row m and 32-column block c (one head's keys):
                  // r = the block's max (0 when every key is masked), out (bf16,
                  // frag_idx with K = ldo) = 2^(s - r), stats[m * ldo / 32 + c] =
                  // {r, sum of those weights in fp32} (gemm_chunk only, one K chunk)
};

struct Epilogue {
  int kind = EPI_STORE;
  void* out = nullptr;
  int ldo = 0;
  int out_f32 = 0;       // 1: fp32 output, 0: bf16
  float* resid = nullptr;
  int ldr = 0;
  int npre = 0, L = 0, hkv = 0, hd = 0;  // EPI_CACHE, EPI_QKV
  int npad = 0;                          // EPI_CACHE, EPI_QKV: key rows per block (npre rounded up)
  int nq = 0;                            // EPI_QKV: query columns
  void* kout = nullptr;                  // EPI_QKV
  void* vout = nullptr;                  // EPI_QKV
  long kv_bs = 0;                        // EPI_QKV: elements between batches of K (and V) blocks
  // W2A8 output scaling: y = bf16(float(acc) * (alpha[m] * beta[n])) before the epilogue
  const float* alpha = nullptr;
  const float* beta = nullptr;
  int32_t* acc_out = nullptr;  // optional raw int32 accumulators [M][N]
  int out_frag = 0;  // bf16 output in fragment layout (frag_idx with K = ldo) instead of rows
  // EPI_CACHE, bf16, one observation: the values also go to vcopy in frag_idx
  // order, block (l, h) of npad * hd elements at (l * hkv + h) * npad * hd (the
  // operand order the absorbed cross-attention products contract over hd in)
  void* vcopy = nullptr;
  // EPI_SCORES: per-row block maxima and sums, visible keys
  float* stats = nullptr;
  const int* klen = nullptr;
  // RMSNorm folded into a product (gemm_chunk, one K chunk): when rss is set,
  // output row m is first scaled by 1 / sqrt(S_m / rdim + reps), S_m the sum
  // of row m's nss partial sums of squares in rss as gemm_chunk_resnorm lays
  // them out (nss = 8, 16, 32 or 64): the norm factor of the row the
  // unnormalised A operand came from
  const float* rss = nullptr;
  int nss = 0, rdim = 0;
  float reps = 0.f;
};

// C = A[M,K] W[N,K]^T, bf16 operands, fp32 accumulation on MFMA, for any row
// count with A ([M][K], rows padded to a multiple of 16) and W ([N][K]) both in
// the fragment layout of common.h, on 288-row tiles.  K % 64 == 0, N % 32 == 0;
// all kinds; STORE and GEGLU need ldo % 4 == 0, RESID ldr % 4 == 0; out_frag
// with bf16 GEGLU or CACHE only.  `splits` > 1 splits K: fp32 partials
// [split][M][N] in `ws`, summed in a fixed order by a reduction (finishing
// kinds) or left for the caller (PARTIAL).  `splits` <= 0 picks a count that
// fills the chip (gemm_frag_splits of them).
hipError_t gemm_frag(const uint16_t* Af, const uint16_t* Wf, int M, int N, int K, const Epilogue& epi,
                     int splits, float* ws, hipStream_t s);
// K splits gemm_frag uses for a product of this shape and epilogue kind (the
// split-K partials of a PARTIAL product, the workspace any other kind needs).
int gemm_frag_splits(int M, int N, int K, int splits, int kind = EPI_PARTIAL);
// True when gemm_frag (with `splits` <= 0) runs a product of this shape and
// kind as whole-K row tiles: no partials, every output stored once by its
// owner (QKV and RESID kinds at a few hundred rows).
bool gemm_frag_rowtile(int M, int N, int K, int kind);

// Number of K splits gemm_chunk actually uses for a request of `splits`.
int gemm_chunk_splits(int K, int splits);

// The same contraction for at most 64 rows with A and W ([N][K]) both in the
// fragment layout of common.h: every load of a wave is one contiguous 1 KB
// block.  A holds 16 rows when M <= 16, 32 when M <= 32, else 64; rows past M
// are read but their results never stored.  K % 32 == 0, N % 32 == 0; kinds
// STORE, PARTIAL, GEGLU, QKV and CACHE (out_frag honoured); split sums of the
// finishing kinds go through a fixed-order reduction; partials as gemm_frag
// (gemm_chunk_splits of them).  `prefetch` (optional) appends extra workgroups that read weights
// of later kernels, as for the row kernels.
hipError_t gemm_chunk(const uint16_t* Af, const uint16_t* Wf, int M, int N, int K, const Epilogue& epi,
                      int splits, float* ws, hipStream_t s, const Prefetch* prefetch = nullptr);
// Residual-updating product of at most 64 rows with RMSNorm's inputs for the
// next product: h[m][n] += (A W^T)[m][n] for m < M (fp32 rows, ldh apart), and,
// when gain is set, xb = bf16(h_new * (1 + gain[n])) in the fragment layout
// (K = N) and, per row, N / 16 partial sums of h_new^2 over 16 columns each
// in ss (N / 16 * 64 floats, laid out [x][64][N / 128] by the XCD x whose
// workgroups wrote them, so every line of ss, h and xb is written from one
// L2); the next product scales its rows by the norm factor (Epilogue::rss).
// A workgroup owns 16 rows x 16 columns over the whole K range (eight waves
// split K, summed in wave order), so each output has one owner and the
// results never depend on timing.  A and W in the fragment layout; M <= 64,
// N % 128 == 0, N <= 1024, K % 32 == 0, K <= 4096.
hipError_t gemm_chunk_resnorm(const uint16_t* Af, const uint16_t* Wf, int M, int N, int K, float* h, int ldh,
                              const float* gain, uint16_t* xb, float* ss, hipStream_t s, const Prefetch* prefetch);
// The Prefetch `group` for the weights of gemm_chunk_resnorm (0: ungrouped).
size_t gemm_chunk_resnorm_group_bytes(int N, int K);
// The residual update of an absorbed cross-attention sublayer, as
// gemm_chunk_resnorm with A = the softmax weights of gemm_chunk's EPI_SCORES
// output (pw: 2^(s - r) per 32-key block, stats: {r, block sum} per row and
// block, K = Hq * npad columns, bph = npad / 32 blocks per head): each block's
// products are scaled by 2^(r - R) / L, R and L the max and weight sum over its
// head's blocks, before they are summed, so h += softmax(S) Wvo^T head by head.
// K % 32 == 0, K <= 4096, bph <= 16, K / 32 / bph <= 32 heads.
hipError_t gemm_chunk_probres(const uint16_t* pw, const float* stats, int bph, const uint16_t* Wf, int M, int N,
                              int K, float* h, int ldh, const float* gain, uint16_t* xb, float* ss, hipStream_t s,
                              const Prefetch* prefetch);
// Products of the absorbed cross attention for one observation and every
// expert layer (bf16, fragment layouts; Np keys per head block, a multiple of
// 32; qe = Hq * hd; layer l's blocks at l * the per-layer stride):
//   wqk[l] [Hq Np][d_e]: row j Np + t = sl2 * sum_d K_l,g(j)[t][d] Wq_l[j hd + d][:]
//     (k: cache keys, frag_idx order; wqT: Wq_l transposed, [d_e][qe]);
//   wvo[l] [d_e][Hq Np]: column j Np + t = sum_d Wo_l[:][j hd + d] V_l,g(j)[t][d]
//     (v: cache values in frag_idx order; wo: [d_e][qe]).
// g(j) = j * Hkv / Hq.  k_ls / v_ls: elements between layers of k / v; wq_ls /
// wo_ls: between layers of wqT / wo; out_ls: between layers of wqk and wvo.
struct AbsorbP {
  const uint16_t *k, *v, *wqT, *wo;
  uint16_t *wqk, *wvo;
  long k_ls, v_ls, wq_ls, wo_ls, out_ls;
  int L, Hq, Hkv, hd, Np, d_e;
  float sl2;
};
hipError_t absorb_products(const AbsorbP& p, hipStream_t s);
// Bytes of fragment-layout weight that one column group of gemm_chunk reads
// (the workgroup grid's x index), or 0 when the groups do not map to XCDs
// round robin (grid width not a multiple of 8): the `group` of a Prefetch.
size_t gemm_chunk_group_bytes(int M, int N, int K, int kind, int splits);
// row-major bf16 [N][K] -> fragment layout (N % 16 == 0, K % 32 == 0)
hipError_t frag_pack(const uint16_t* src, int N, int K, uint16_t* dst, hipStream_t s);
// row-major bf16 [R][C] -> fragment layout of its transpose [C][R] (C % 16 == 0, R % 32 == 0)
hipError_t frag_pack_t(const uint16_t* src, int R, int C, uint16_t* dst, hipStream_t s);

// Same contraction in fp32 on the vector ALU (fp32 workloads); K % 16 == 0.
hipError_t gemm_f32(const float* A, int lda, const float* W, int ldw, int M, int N, int K,
                    const Epilogue& epi, hipStream_t s);

// Ternary W2A8: acc = a[M,K] q[N,K]^T in int32 on int8 MFMA, q in the library's
// packed layout (see w2a8.hip); y = bf16(float(acc) * alpha[m] * beta[n]) into the
// epilogue (epi.alpha / epi.beta must be set).  K % 128 == 0, N % 32 == 0.
// epi.kind is EPI_STORE, EPI_RESID or EPI_GEGLU.  With `work` the K range may be
// split over several workgroups per output tile (when the tiles alone leave CUs
// idle): ws holds their int32 partial sums (w2a8_part_bytes), cnt one counter
// per tile (w2a8_counters), zero before the first launch and left zero by
// every launch.  Launches sharing one `work` must not overlap.
struct W2A8Work {
  int* ws = nullptr;
  size_t ws_bytes = 0;
  unsigned* cnt = nullptr;
  int ncnt = 0;
};
size_t w2a8_part_bytes(int M, int N);
int w2a8_counters(int M, int N);
hipError_t gemm_w2a8(const int8_t* a, int lda, const uint32_t* qp, int M, int N, int K,
                     const Epilogue& epi, hipStream_t s, const W2A8Work* work = nullptr);

// Same with one scale beta for every output channel (epi.beta ignored).
hipError_t gemm_w2a8_scalar(const int8_t* a, int lda, const uint32_t* qp, int M, int N, int K,
                            const Epilogue& epi, float beta_scalar, hipStream_t s, const W2A8Work* work = nullptr);

// The same on the vector ALU (v_dot4_i32_i8), bf16 STORE epilogue and/or raw
// accumulators only; beta[n] from epi.beta when set, else beta_scalar.  K % 64 == 0.
hipError_t gemm_w2a8_dot4(const int8_t* a, int lda, const uint32_t* qp, int M, int N, int K,
                          const Epilogue& epi, float beta_scalar, hipStream_t s);

// Canonical packed ternary [N][K/4] bytes -> library layout; flags[0] |= 1 on a code 3.
hipError_t ternary_repack(const uint8_t* canon, int N, int K, uint32_t* out, int* flags, hipStream_t s);

// Fixed device scratch of the allocation-free ternary GEMM entry point
// (w2a8.hip): kW2A8ScratchBytes bytes per device, the repacked words first and
// a 256-byte flag area at the end.  w2a8_scratch returns its device address on
// the current device (looked up once per device).
constexpr size_t kW2A8ScratchBytes = (size_t)16 << 20;
constexpr size_t kW2A8FlagBytes = 256;
constexpr int kMaxDevices = 64;
hipError_t w2a8_scratch(void** ptr);

// ------------------------------------------------------------------ row kernels
// Row-wise residual update and RMSNorm: for each row m,
//   h[m] += sum_s part[s][m]           (if nsplit > 0; part is [nsplit][M][N] fp32)
//   u = h[m] / sqrt(mean(h[m]^2) + eps) * (1 + gain)
// and u is written as bf16 / fp32 (u_out), or quantized per Eq. 4 to int8 codes
// (q_out) with its scale (alpha_out).  Any of the outputs may be null.
// With u_frag the bf16 u goes out in the fragment layout (K = N) instead of rows.
// `prefetch` (nullable) adds workgroups that read the next kernel's weights once.
hipError_t resid_norm(float* h, int ldh, const float* part, int nsplit, int M, int N,
                      const float* gain, float eps, void* u_out, int u_f32, int ldu,
                      int8_t* q_out, float* alpha_out, hipStream_t s, int u_frag = 0,
                      const Prefetch* prefetch = nullptr);

// Eq. 4 per-row quantization of fp32 rows (x: [M][ldx], K valid columns).
hipError_t quantize_rows(const float* x, int ldx, int M, int K, int8_t* a, float* alpha, hipStream_t s);

// ------------------------------------------------------------------ attention
struct AttnArgs {
  const void* q; long q_bs, q_hs, q_rs;   // element strides: batch, head, row
  const void* k; long k_bs, k_hs, k_rs;
  const void* v; long v_bs, v_hs, v_rs;
  void* o; long o_bs, o_rs;               // output head j at column j * hd
  int B, Nq, Nk, Hq, Hkv, hd;
  // optional second key/value source, appended after the first Nk keys in one
  // softmax (joint attention): Nk2 keys laid out like the first source
  const void* k2; long k2_bs, k2_hs, k2_rs;
  const void* v2; long v2_bs, v2_hs, v2_rs;
  int Nk2;
  int o_f32;                              // 1: fp32 output, 0: bf16
  int o_frag;                             // bf16 output in fragment layout: row b * Nq + q, K = Hq * hd
  Prefetch pf;                            // attention_chunk: extra workgroups warming the next weights
  // key padding (Eq. 2, M = -inf): batch b sees only its first klen[b] keys of
  // the first source (klen2[b] of the second); device arrays of B entries in
  // [1, Nk] (or [1, Nk2]), or null when every key is visible
  const int* klen;
  const int* klen2;
};
// softmax(Q K^T / sqrt(hd) + M) V per head, M the key padding above; bf16 inputs on MFMA (hd in 64..256)
hipError_t attention_bf16(const AttnArgs& a, hipStream_t s);
// The same for short query sets with K and V in the MFMA operand orders of
// common.h (frag_idx / vfrag_idx per batch-and-head block of k_bs / k_hs
// elements, key rows padded to a multiple of 32 with zero values); Q rows as
// above (k_rs, v_rs unused); bf16 output only.
hipError_t attention_chunk(const AttnArgs& a, hipStream_t s);
// fp32 inputs on the vector ALU (small shapes)
hipError_t attention_f32(const AttnArgs& a, hipStream_t s);

// ------------------------------------------------------------------ expert pieces
// Zero the last `tail` 16-bit elements of each of nblk blocks of `blk` elements
// (the padding key rows of fragment-ordered K/V blocks); tail, blk % 8 == 0.
hipError_t zero_tails(void* base, long nblk, long blk, int tail, hipStream_t s);
// Row kernel of the solver loop: the velocity head and Euler update of step
// k_head (skipped when < 0), then the embedding of step k_embed with the first
// layer's RMSNorm (skipped when < 0).  E is read by the head, Eout written by
// the embedding (they may alias).
struct StepRows {
  const float* E = nullptr;
  float* Eout = nullptr;
  float* X = nullptr;
  int M = 0, d_e = 0, d_a = 0;
  float eps = 0.f;
  const float* gain_f = nullptr;  // final expert norm gain (head)
  const void* w_out = nullptr;
  const void* w_in = nullptr;
  const float* gain_1 = nullptr;  // first expert layer's norm gain (embedding)
  void* u = nullptr;
  int u_f32 = 0, u_frag = 0;
  const float* sched = nullptr;
  int k_head = -1, k_embed = -1;
  Prefetch pf;
};
hipError_t step_rows(const StepRows& a, int w_f32, hipStream_t s);
// ------------------------------------------------------------------ persistent solver step
// One solver step of the bf16 cross-attention expert for at most 64 chunk rows
// as one persistent kernel (fused.hip): the same tiles and summation orders as
// the kernel chain of run_steps, phases separated by grid barriers.  Byte
// sizes bound every coherent access (buffer resources); all below 2 GB.
struct FusedStepP {
  int M, B, H, Hp, N, Np;               // chunk rows, batch, chunk tokens (padded), prefix tokens (padded)
  int d_e, d_a, F, L, Hq, Hkv, D;       // expert shapes, D = hd_e
  int qe, qkve, nrb;                    // query width, fused projection width, 16-row attention blocks
  float eps;
  int k_head, k_embed;                  // row phase at the start (either may be < 0)
  int trailing_head, k_tail;            // last step: head of step k_tail after the last layer
  unsigned gen, gen_tail;               // barrier generations of this launch
  int kc_qkv, kc_q, kc_gu, kc_o, kc_d;  // K chunk (elements) of each GEMM, as gemm_chunk plans it
  int s_o, s_d;                         // K splits of the O and down projections
  int spw_qkv, spw_q, spw_gu, spw_o, spw_d;  // k-steps per wave
  const char* ew;                       // expert weight arena, layer l at ew + l * ew_layer
  long ew_layer, off_qkv, off_os, off_qc, off_oc, off_gu, off_d;
  const float* egains;                  // [L][3][d_e]: a1, a2, a3
  const float* w_ef;
  const uint16_t* w_out;
  const uint16_t* w_in;
  const float* sched;
  const uint16_t* cache;                // [B][L][2][Hkv][Np][D], MFMA operand orders
  const int* klen;                      // visible prefix keys per observation
  float* E;
  float* X;
  uint16_t *u, *q, *kc, *vc, *attn, *eq, *g;
  float* part;
  uint32_t bytes_E, bytes_X, bytes_u, bytes_q, bytes_kv, bytes_attn, bytes_g, bytes_part, bytes_cache;
  unsigned* bar;                        // fused_barrier_words(L) words, zeroed per solver run
  unsigned* err;                        // bit 0: a barrier wait gave up
  int nwg;                              // compute workgroups (all resident)
};
long fused_barrier_words(int L);
hipError_t fused_zero(unsigned* bar, long words, hipStream_t s);
// workgroups of k_fused_step that fit on one CU for head width D and M chunk rows
int fused_occupancy(int D, int M);
// launch one step: nwg compute workgroups, plus nwg shadow workgroups if `shadows`
hipError_t fused_step(const FusedStepP& p, int shadows, hipStream_t s);
// K split plan of gemm_chunk: number of chunks and chunk length in elements
void gemm_chunk_plan(int K, int splits, int* used, int* kchunk);

// Per-observation prefix lengths into a device array: dst[b] = len[b] (host
// values, passed to the kernel by value in groups of 64), or N for every b
// when len is null.
hipError_t set_lengths(int* dst, const int32_t* len, int B, int N, hipStream_t s);
// dst = src for the [B][N][d] prefix rows (src fp32, or bf16 widened to fp32
// when src_bf16), with the rows of observation b past its length lens[b]
// (device; null: every row kept) written as zeros.
hipError_t copy_prefix_rows(const void* src, int src_bf16, float* dst, int B, int N, int d, const int* lens,
                            hipStream_t s);
// dst = src (fp32), or bf16(src) when out_bf16
hipError_t copy_out(const float* src, void* dst, long n, int out_bf16, hipStream_t s);
hipError_t copy_f32(const float* src, float* dst, long n, hipStream_t s);
// fp32 -> bf16 conversion of a weight tensor
hipError_t f32_to_bf16(const float* src, uint16_t* dst, long n, hipStream_t s);

}  // namespace vla
