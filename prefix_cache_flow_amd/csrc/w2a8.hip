// Ternary W2A8 GEMM of the paper's §III-D, Eq. 4:
//   acc[m][n] = sum_j a[m][j] q[n][j]   (int8 activations x ternary weights, int32)
//   y[m][n]   = bf16(float(acc) * (alpha[m] * beta[n]))   (nearest, ties to even)
//
// Weight layout inside the library: one 32-bit word per 16 consecutive inputs of
// an output row, input e = 4i + b of the group at bits 8b + 2i (code = q + 1).
// With that order, (word >> 2i) & 0x03030303 holds inputs 4i..4i+3 in its four
// bytes, and one byte permute against the table {-1, 0, +1} turns the 2-bit
// codes into int8 lanes: a 16-input MFMA fragment comes out of one word with
// four shifts, four masks and four permutes.  The canonical format of the C ABI
// (input 4j + i in bits 2i of byte j) is converted to this order once, when the
// model is created.
//
// Tiles: 64 activation rows x 128 output channels per workgroup of eight
// waves (two per SIMD, four with the two workgroups a CU holds), 256-input K
// slices (128 when 256 does not divide K), 32x32x32 int8 MFMA.  Each wave
// accumulates 64 rows x 32 channels over half of every slice; the halves meet
// once through LDS, after which each wave holds one 32 x 32 block and all
// eight share the epilogue.  The activation slice is
// staged in LDS as int8; the weight slice is staged *packed* (2 bits per
// weight, a quarter of the int8 bytes) and unpacked in registers right before
// the MFMA.  When the output tiles alone would leave CUs idle, the K range of
// a tile is split over up to three workgroups whose int32 partial sums meet in
// a workspace (exact in any order).
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace vla {

struct W2A8P {
  const int8_t* a;
  int lda;
  const uint32_t* q;  // [N][K/16] words
  int M, N, K, nM, nN;
  Epilogue epi;
  float beta_scalar;
  int S = 1;               // K splits per output tile (1: no partial sums)
  int* ws = nullptr;       // S > 1: partial sums, kW2A8PartInts per (tile, split)
  unsigned* cnt = nullptr; // S > 1: per-tile arrival counters, zero between launches
};

__device__ __forceinline__ i32x4_t unpack16(uint32_t w) {
  i32x4_t r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = (int)__builtin_amdgcn_perm(0u, 0x000100FFu, (w >> (2 * i)) & 0x03030303u);
  return r;
}

namespace {
constexpr int kBM = 64, kBN = 128;       // output tile
constexpr int kPartInts = kBM * kBN;     // one tile's partial sums
constexpr int kSC1 = 16;                 // cache policy bits of device-scope coherent loads and stores
}  // namespace

// Epilogue of one wave: row half `own` (rows m0 + 32 own + mfma32_row(q, lane))
// of channel half c, both 32-channel groups g (channels n0 + 64 c + 32 g +
// lane % 32).  The kind, the int32 copy and the output type are template
// parameters, so each kernel carries one short straight-line store path (these
// kernels start with a cold instruction cache), and every load (residual
// values) is issued before the first store: loads and stores retire through one
// counter here, so a load placed after a store would wait for that store's
// round trip too.
template <int KIND, bool ACC, bool F32, int GB>
__device__ __forceinline__ void w2a8_epilogue(const W2A8P& p, const i32x16_t (&fin)[GB], int own, int col0, int lane,
                                              int m0, int n0, const float* s_al, const float* s_be) {
  const Epilogue& e = p.epi;
  const int mb = m0 + own * 32, nb = n0 + col0 + (lane & 31);
  float al[16], be[GB], rv[GB][16];
#pragma unroll
  for (int q = 0; q < 16; ++q) al[q] = s_al[own * 32 + mfma32_row(q, lane)];
#pragma unroll
  for (int g = 0; g < GB; ++g) be[g] = s_be[col0 + g * 32 + (lane & 31)];
  if (KIND == EPI_RESID) {
#pragma unroll
    for (int g = 0; g < GB; ++g)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int m = mb + mfma32_row(q, lane), n = nb + g * 32;
        rv[g][q] = (m < p.M && n < p.N) ? e.resid[(long)m * e.ldr + n] : 0.f;
      }
  }
#pragma unroll
  for (int g = 0; g < GB; ++g) {
    const int n = nb + g * 32;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int m = mb + mfma32_row(q, lane);
      const bool ok = m < p.M && n < p.N;
      if (ACC && ok) e.acc_out[(long)m * p.N + n] = fin[g][q];
      const float y = ok ? bf2f(f2bf((float)fin[g][q] * (al[q] * be[g]))) : 0.f;
      if (KIND == EPI_GEGLU) {
        const float other = __shfl_xor(y, 16, 64);
        if (!(lane & 16) && ok) {
          const float v = gelu_erf(y) * other;
          const long o = (long)m * e.ldo + (n >> 5) * 16 + (lane & 15);
          if (F32) ((float*)e.out)[o] = v; else ((bf16_t*)e.out)[o] = f2bf(v);
        }
      } else if (KIND == EPI_RESID) {
        if (ok) e.resid[(long)m * e.ldr + n] = rv[g][q] + y;
      } else if (ok && e.out) {
        const long o = (long)m * e.ldo + n;
        if (F32) ((float*)e.out)[o] = y; else ((bf16_t*)e.out)[o] = f2bf(y);
      }
    }
  }
}

// One 64 x 128 output tile (or one K split of it) per workgroup of eight
// waves.  Wave (cg, kh) = (w & 3, w >> 2) accumulates all 64 rows of channel
// group cg (32 channels) over the k half kh of every slice: each weight word
// is unpacked by exactly one wave and feeds two MFMAs (the two 32-row blocks,
// whose accumulators alternate, so consecutive MFMAs do not wait on each
// other).  At the end the two k halves meet once through LDS: wave kh keeps
// row block kh and hands the other to its partner (int32: exact in any order),
// so all eight waves finish one 32 x 32 block each and share the epilogue.
template <int BK, int KIND, bool ACC>
__global__ __launch_bounds__(512, 4) void k_gemm_w2a8(W2A8P p) {
  constexpr int BM = kBM, BN = kBN, LDA = BK + 16, LDW = BK / 16 + 1;
  constexpr int KPW = BK / 32 / 2;                // MFMA k-steps per wave and slice (a half)
  constexpr int AV = BM * BK / 16 / 512;          // 16-byte activation vectors per thread and slice
  constexpr int WW = BN * BK / 16 / 512;          // weight words per thread and slice (4 or 2)
  constexpr int STAGE = 2 * BM * LDA + 2 * BN * LDW * 4;
  constexpr int XCH = 8 * 16 * 64 * 4;            // eight waves' handed-over blocks (16 ints a lane)
  constexpr int LDS = STAGE > XCH ? STAGE : XCH;
  static_assert(AV >= 1 && (WW == 4 || WW == 2) && KPW >= 1, "slice shape");
  typedef __attribute__((__vector_size__(WW * sizeof(uint32_t)))) uint32_t wvec_t;
  __shared__ __attribute__((aligned(16))) unsigned char lds[LDS];
  __shared__ float s_al[BM], s_be[BN];
  __shared__ unsigned s_last;
  int8_t(*sA)[BM * LDA] = (int8_t(*)[BM * LDA])lds;
  uint32_t(*sW)[BN * LDW] = (uint32_t(*)[BN * LDW])(lds + 2 * BM * LDA);
  int* xch = (int*)lds;

  // work item -> (tile, split); consecutive items share an XCD (linear id mod 8),
  // so the splits of a tile and the row tiles of one weight column meet in one L2
  const int W = p.nM * p.nN * p.S, L = blockIdx.x;
  const int wk = (W % 8 == 0) ? (L % 8) * (W / 8) + L / 8 : L;
  const int sp = wk % p.S, tile = wk / p.S;
  const int tm = tile % p.nM, tn = tile / p.nM;
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cg = wid & 3, kh = wid >> 2;  // channel group of 32, k half of every slice
  const int KW = p.K / 16;                // words per weight row
  const int ns = p.K / BK, s_lo = sp * ns / p.S, nsl = (sp + 1) * ns / p.S - s_lo;
  const Epilogue& e = p.epi;
  if (tid < BM) s_al[tid] = e.alpha[min(m0 + tid, p.M - 1)];
  else if (tid < BM + BN) s_be[tid - BM] = e.beta ? e.beta[min(n0 + tid - BM, p.N - 1)] : p.beta_scalar;

  struct Regs { u32x4_t a[AV]; wvec_t w; };
  constexpr int AR = BK / 16, WR = BK / 16 / WW;  // vectors per activation row, per weight row
  auto gload = [&](Regs& g, int i) {
    const int k0 = (s_lo + min(i, nsl - 1)) * BK;  // past the end: the last slice again (never used)
#pragma unroll
    for (int v0 = 0; v0 < AV; ++v0) {
      const int v = tid + v0 * 512, r = v / AR, cc = (v % AR) * 16;
      // rows past the end are clamped to valid ones; their results are never stored
      g.a[v0] = *(const u32x4_t*)(p.a + (long)min(m0 + r, p.M - 1) * p.lda + k0 + cc);
    }
    const int r = tid / WR, cc = (tid % WR) * WW;
    g.w = *(const wvec_t*)(p.q + (long)min(n0 + r, p.N - 1) * KW + k0 / 16 + cc);
  };
  auto sstore = [&](const Regs& g, int buf) {
#pragma unroll
    for (int v0 = 0; v0 < AV; ++v0) {
      const int v = tid + v0 * 512;
      *(u32x4_t*)&sA[buf][(v / AR) * LDA + (v % AR) * 16] = g.a[v0];
    }
    const int r = tid / WR, cc = (tid % WR) * WW;
#pragma unroll
    for (int t = 0; t < WW; ++t) sW[buf][r * LDW + cc + t] = g.w[t];
  };

  i32x16_t acc[2];  // row blocks 0 and 1
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[i][q] = 0;
  auto compute = [&](int buf) {
    i32x4_t af[KPW][2];
    uint32_t wq[KPW];
#pragma unroll
    for (int j = 0; j < KPW; ++j) {
      const int kk = kh * KPW + j;
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[j][i] = __builtin_bit_cast(
            i32x4_t, *(const u32x4_t*)&sA[buf][(i * 32 + (lane & 31)) * LDA + kk * 32 + (lane >> 5) * 16]);
      wq[j] = sW[buf][(cg * 32 + (lane & 31)) * LDW + kk * 2 + (lane >> 5)];
    }
#pragma unroll
    for (int j = 0; j < KPW; ++j) {
      const i32x4_t wf = unpack16(wq[j]);
#pragma unroll
      for (int i = 0; i < 2; ++i) acc[i] = mfma32x32x32_i8(af[j][i], wf, acc[i]);
    }
  };
  // Slice t lives in register set t % NR until it is stored to LDS buffer
  // t % 2 (NR = 3 register sets for 128-input slices, 2 for 256-input ones,
  // which keeps four waves per SIMD within the register file).  Entering step
  // t: slice t in LDS, slices t + 1 .. t + NR in flight.  The scheduling
  // barriers keep the compiler from moving a load or a store across a step
  // boundary: in program order the slice stored at step t is the oldest in
  // flight, so its wait leaves the others outstanding.  Groups of NR steps keep
  // the register-set index static; the LDS buffer index alternates at run
  // time, and steps past the last slice compute nothing.
  constexpr int NR = BK == 256 ? 2 : 3;
  Regs rs[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) gload(rs[i], i);
  sstore(rs[0], 0);
  __syncthreads();
  gload(rs[0], NR);
#define W2A8_STEP(J)                                  \
  if ((J) < NR) {                                     \
    const int t = t0 + (J);                           \
    if (t < nsl) compute(t & 1);                      \
    __builtin_amdgcn_sched_barrier(0);                \
    sstore(rs[((J) + 1) % NR], (t + 1) & 1);          \
    __syncthreads();                                  \
    gload(rs[((J) + 1) % NR], t + NR + 1);            \
    __builtin_amdgcn_sched_barrier(0);                \
  }
  for (int t0 = 0; t0 < nsl; t0 += NR) {
    W2A8_STEP(0) W2A8_STEP(1) W2A8_STEP(2)
  }
#undef W2A8_STEP

  // The two k halves: wave kh keeps row block kh; the other block goes to the
  // partner wave through LDS (16-byte chunks, lane-major).  fin is copied out
  // of the accumulators by static indices in each branch.
  i32x16_t fin[1], give;
  if (kh == 0) { fin[0] = acc[0]; give = acc[1]; }
  else { fin[0] = acc[1]; give = acc[0]; }
  __syncthreads();  // the staging buffers are free from here on
#pragma unroll
  for (int h4 = 0; h4 < 4; ++h4)
    *(i32x4_t*)(xch + ((wid * 4 + h4) * 64 + lane) * 4) =
        i32x4_t{give[4 * h4], give[4 * h4 + 1], give[4 * h4 + 2], give[4 * h4 + 3]};
  __syncthreads();
  {
    const int partner = wid ^ 4;
#pragma unroll
    for (int h4 = 0; h4 < 4; ++h4) {
      const i32x4_t v = *(const i32x4_t*)(xch + ((partner * 4 + h4) * 64 + lane) * 4);
#pragma unroll
      for (int q = 0; q < 4; ++q) fin[0][4 * h4 + q] += v[q];
    }
  }
  // this wave now holds row block kh of channel group cg: slot wid of a
  // tile's partial sums below

  if (p.S > 1) {
    // K split: every split stores its sums with device-scope coherent stores
    // (the XCDs' L2s are not coherent with one another), waits for their
    // acknowledgement, then counts itself in; the last to arrive adds the other
    // splits' sums (loaded the same way), resets the counter for the next
    // launch and runs the epilogue.  No workgroup ever waits on another.
    const uint32_t bytes = (uint32_t)((size_t)W * kPartInts * 4);
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(p.ws, (short)0, (int)bytes, 0x00020000);
    auto off = [&](int split, int h4) {
      return (uint32_t)(((size_t)(tile * p.S + split) * kPartInts + (wid * 4 + h4) * 256 + lane * 4) * 4);
    };
#pragma unroll
    for (int h4 = 0; h4 < 4; ++h4)
      __builtin_amdgcn_raw_buffer_store_b128(
          __builtin_bit_cast(u32x4_t, i32x4_t{fin[0][4 * h4], fin[0][4 * h4 + 1], fin[0][4 * h4 + 2], fin[0][4 * h4 + 3]}), r,
          off(sp, h4), 0, kSC1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) {
      const unsigned old = __hip_atomic_fetch_add(p.cnt + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = old + 1 == (unsigned)p.S;
      if (s_last) __hip_atomic_store(p.cnt + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!s_last) return;
    for (int o = 0; o < p.S; ++o) {
      if (o == sp) continue;
      u32x4_t in[4];
#pragma unroll
      for (int h4 = 0; h4 < 4; ++h4) in[h4] = __builtin_amdgcn_raw_buffer_load_b128(r, off(o, h4), 0, kSC1);
#pragma unroll
      for (int q = 0; q < 16; ++q) fin[0][q] += (int)in[q / 4][q % 4];
    }
  }
  if (e.out_f32) w2a8_epilogue<KIND, ACC, true, 1>(p, fin, kh, cg * 32, lane, m0, n0, s_al, s_be);
  else w2a8_epilogue<KIND, ACC, false, 1>(p, fin, kh, cg * 32, lane, m0, n0, s_al, s_be);
}

size_t w2a8_part_bytes(int M, int N) {
  const size_t tiles = (size_t)((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
  return tiles * 3 * kPartInts * 4;
}

int w2a8_counters(int M, int N) { return ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN); }

namespace {
int cu_count() {
  static int cached[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}
}  // namespace

hipError_t gemm_w2a8_scalar(const int8_t* a, int lda, const uint32_t* qp, int M, int N, int K, const Epilogue& epi,
                            float beta_scalar, hipStream_t s, const W2A8Work* work) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (K % 128 || N % 32 || !epi.alpha) return hipErrorInvalidValue;
  if (epi.kind != EPI_STORE && epi.kind != EPI_RESID && epi.kind != EPI_GEGLU) return hipErrorInvalidValue;
  W2A8P p{a, lda, qp, M, N, K, (M + kBM - 1) / kBM, (N + kBN - 1) / kBN, epi, beta_scalar};
  // 256-wide K slices when they divide K: a weight row's slice is then 64
  // contiguous bytes and each wave gets two k-steps per slice
  const bool wide = K % 256 == 0;
  // K splits while the tiles alone leave CUs idle: at most three, at least four
  // slices each, and only with room for the partial sums and counters
  const int tiles = p.nM * p.nN, ns = K / (wide ? 256 : 128);
  int S = 1;
  if (work && work->ws && work->cnt && work->ncnt >= tiles) {
    S = std::min(3, std::max(1, cu_count() / tiles));
    while (S > 1 && (ns / S < 4 || (size_t)tiles * S * kPartInts * 4 > work->ws_bytes)) --S;
    if (S > 1) { p.S = S; p.ws = work->ws; p.cnt = work->cnt; }
  }
  const dim3 grid(tiles * S), block(512);
  const bool acc = epi.acc_out != nullptr;
#define W2A8_LAUNCH(BK, KIND)                                                                   \
  do {                                                                                          \
    if (acc) hipLaunchKernelGGL((k_gemm_w2a8<BK, KIND, true>), grid, block, 0, s, p);           \
    else hipLaunchKernelGGL((k_gemm_w2a8<BK, KIND, false>), grid, block, 0, s, p);              \
  } while (0)
#define W2A8_KINDS(BK)                                                                          \
  do {                                                                                          \
    if (epi.kind == EPI_RESID) W2A8_LAUNCH(BK, EPI_RESID);                                      \
    else if (epi.kind == EPI_GEGLU) W2A8_LAUNCH(BK, EPI_GEGLU);                                 \
    else W2A8_LAUNCH(BK, EPI_STORE);                                                            \
  } while (0)
  if (wide) W2A8_KINDS(256);
  else W2A8_KINDS(128);
#undef W2A8_KINDS
#undef W2A8_LAUNCH
  return hipGetLastError();
}

hipError_t gemm_w2a8(const int8_t* a, int lda, const uint32_t* qp, int M, int N, int K, const Epilogue& epi,
                     hipStream_t s, const W2A8Work* work) {
  return gemm_w2a8_scalar(a, lda, qp, M, N, K, epi, 0.f, s, work);
}

// The same contraction on the vector ALU with v_dot4_i32_i8 (four int8
// products summed into an int32 per lane and instruction): the counterpart of
// the page's dp4a path, kept to compare against the matrix cores.  Tiles of
// 64 rows x 64 output channels x 64 inputs: the activation slice (int8) and the
// packed weight slice go through LDS, and each thread accumulates 4 rows x 4
// channels, unpacking each weight word once for its four rows.  Integer sums
// are exact, so the accumulators equal the MFMA kernel's bit for bit.
__global__ __launch_bounds__(256) void k_gemm_w2a8_dot4(W2A8P p) {
  constexpr int BM = 64, BN = 64, BK = 64, LDA = BK / 4 + 1, LDW = BK / 16 + 1;  // LDA, LDW in words
  __shared__ uint32_t sA[BM * LDA];
  __shared__ uint32_t sW[BN * LDW];
  const int tm = blockIdx.x % p.nM, tn = blockIdx.x / p.nM;
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x, rg = tid >> 4, cg = tid & 15;
  const int KW = p.K / 16;
  int acc[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[r][j] = 0;
  for (int k0 = 0; k0 < p.K; k0 += BK) {
    // 64 rows x 16 words of activations, 64 channels x 4 words of weights
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int v = tid + i * 256, r = v >> 4, c = v & 15;
      sA[r * LDA + c] = *(const uint32_t*)(p.a + (long)min(m0 + r, p.M - 1) * p.lda + k0 + c * 4);
    }
    {
      const int r = tid >> 2, c = tid & 3;
      sW[r * LDW + c] = p.q[(long)min(n0 + r, p.N - 1) * KW + k0 / 16 + c];
    }
    __syncthreads();
#pragma unroll
    for (int wi = 0; wi < BK / 16; ++wi) {
      uint32_t wv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) wv[j] = sW[(cg * 4 + j) * LDW + wi];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int q[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) q[j] = (int)__builtin_amdgcn_perm(0u, 0x000100FFu, (wv[j] >> (2 * i)) & 0x03030303u);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int av = (int)sA[(rg * 4 + r) * LDA + wi * 4 + i];
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[r][j] = __builtin_amdgcn_sdot4(av, q[j], acc[r][j], false);
        }
      }
    }
    __syncthreads();
  }
  // scales first, then stores (a load after a store would wait for the store)
  const Epilogue& e = p.epi;
  float al[4], bt[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) al[r] = e.alpha[min(m0 + rg * 4 + r, p.M - 1)];
#pragma unroll
  for (int j = 0; j < 4; ++j) bt[j] = e.beta ? e.beta[min(n0 + cg * 4 + j, p.N - 1)] : p.beta_scalar;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = m0 + rg * 4 + r;
    if (m >= p.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + cg * 4 + j;
      if (n >= p.N) continue;
      if (e.acc_out) e.acc_out[(long)m * p.N + n] = acc[r][j];
      if (e.out) ((bf16_t*)e.out)[(long)m * e.ldo + n] = f2bf((float)acc[r][j] * (al[r] * bt[j]));
    }
  }
}

hipError_t gemm_w2a8_dot4(const int8_t* a, int lda, const uint32_t* qp, int M, int N, int K, const Epilogue& epi,
                          float beta_scalar, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (K % 64 || !epi.alpha || epi.kind != EPI_STORE || epi.out_f32 || (lda % 4)) return hipErrorInvalidValue;
  W2A8P p{a, lda, qp, M, N, K, (M + 63) / 64, (N + 63) / 64, epi, beta_scalar};
  hipLaunchKernelGGL(k_gemm_w2a8_dot4, dim3(p.nM * p.nN), dim3(256), 0, s, p);
  return hipGetLastError();
}

// canonical [N][K/4] bytes -> [N][K/16] words in the library's order
__global__ void k_ternary_repack(const uint8_t* canon, int N, int K, uint32_t* out, int* flags) {
  const long words = (long)N * (K / 16);
  for (long w = blockIdx.x * (long)blockDim.x + threadIdx.x; w < words; w += (long)gridDim.x * blockDim.x) {
    const long row = w / (K / 16), col = w % (K / 16);
    const uint8_t* src = canon + row * (K / 4) + col * 4;
    uint32_t o = 0;
    int bad = 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const uint32_t code = (src[e >> 2] >> (2 * (e & 3))) & 3u;
      bad |= code == 3u;
      o |= code << (8 * (e & 3) + 2 * (e >> 2));
    }
    out[w] = o;
    if (bad) atomicOr(flags, 1);
  }
}

hipError_t ternary_repack(const uint8_t* canon, int N, int K, uint32_t* out, int* flags, hipStream_t s) {
  if (N <= 0 || K <= 0) return hipSuccess;
  if (K % 16) return hipErrorInvalidValue;
  const long words = (long)N * (K / 16);
  const int blocks = (int)std::min<long>((words + 255) / 256, 4096);
  hipLaunchKernelGGL(k_ternary_repack, dim3(blocks), dim3(256), 0, s, canon, N, K, out, flags);
  return hipGetLastError();
}

// ------------------------------------------------------------------ fixed scratch
// Device memory of the allocation-free ternary GEMM entry point: the repacked
// weight words followed by the invalid-code flag word.  The array is part of
// the code object, so every device the library runs on holds its own copy from
// the moment the module is loaded on it until the process ends; calls on one
// device share (and overwrite) it.  Its name is only a host-side handle: host
// code uses the device address that hipGetSymbolAddress returns, looked up once
// per device with that device current.
static __device__ __align__(256) unsigned char scratch[kW2A8ScratchBytes];

hipError_t w2a8_scratch(void** ptr) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace vla
