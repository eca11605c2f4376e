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
// Tiles: 64 activation rows x 128 output channels x 128 inputs per slice,
// four waves of 64 x 32 on the 32x32x32 int8 MFMA (a wave's unpacked weight
// fragment serves both 32-row halves).  The activation slice is
// staged in LDS as int8; the weight slice is staged *packed* (2 bits per weight,
// a quarter of the int8 bytes) and unpacked in registers right before the MFMA.
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
};

__device__ __forceinline__ i32x4_t unpack16(uint32_t w) {
  i32x4_t r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = (int)__builtin_amdgcn_perm(0u, 0x000100FFu, (w >> (2 * i)) & 0x03030303u);
  return r;
}

__device__ __forceinline__ float w2a8_scale(const W2A8P& p, int m, int n, int acc) {
  const float b = p.epi.beta ? p.epi.beta[n] : p.beta_scalar;
  const float s = p.epi.alpha[m] * b;
  return bf2f(f2bf((float)acc * s));
}

template <int BK>
__global__ __launch_bounds__(256) void k_gemm_w2a8(W2A8P p) {
  constexpr int BM = 64, BN = 128, LDA = BK + 16, LDW = BK / 16 + 1;
  constexpr int AV = BM * BK / 16 / 256;  // 16-byte activation vectors per thread and slice
  constexpr int WV = BN * BK / 64 / 256;  // 4-word weight vectors per thread and slice
  __shared__ __attribute__((aligned(16))) int8_t sA[2][BM * LDA];
  __shared__ uint32_t sW[2][BN * LDW];
  const int nt = p.nM * p.nN, L = blockIdx.x;
  const int tile = (nt % 8 == 0) ? (L % 8) * (nt / 8) + L / 8 : L;
  const int tm = tile % p.nM, tn = tile / p.nM;
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int KW = p.K / 16;  // words per weight row

  // Two register sets, each filled two slices before its trip to LDS, so a
  // slice's global loads have two slices of work to land behind.
  const int ns = p.K / BK;
  struct Regs { u32x4_t a[AV], w[WV]; };
  constexpr int AR = BK / 16, WR = BK / 64;  // vectors per activation row, per weight row
  auto gload = [&](Regs& g, int sl) {
    const int k0 = min(sl, ns - 1) * BK;  // past the end: the last slice again (never used)
#pragma unroll
    for (int i = 0; i < AV; ++i) {
      const int v = tid + i * 256, r = v / AR, c = (v % AR) * 16;
      // rows past the end are clamped to valid ones; their results are never stored
      g.a[i] = *(const u32x4_t*)(p.a + (long)min(m0 + r, p.M - 1) * p.lda + k0 + c);
    }
#pragma unroll
    for (int i = 0; i < WV; ++i) {
      const int v = tid + i * 256, r = v / WR, c = (v % WR) * 4;
      g.w[i] = *(const u32x4_t*)(p.q + (long)min(n0 + r, p.N - 1) * KW + k0 / 16 + c);
    }
  };
  auto sstore = [&](const Regs& g, int buf) {
#pragma unroll
    for (int i = 0; i < AV; ++i) {
      const int v = tid + i * 256;
      *(u32x4_t*)&sA[buf][(v / AR) * LDA + (v % AR) * 16] = g.a[i];
    }
#pragma unroll
    for (int i = 0; i < WV; ++i) {
      const int v = tid + i * 256, r = v / WR, c = (v % WR) * 4;
#pragma unroll
      for (int t = 0; t < 4; ++t) sW[buf][r * LDW + c + t] = g.w[i][t];
    }
  };

  i32x16_t acc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0;
  // wave w owns output channels 32 w .. 32 w + 31 for all 64 rows: each
  // weight word it unpacks feeds two MFMAs (the two 32-row halves)
  auto compute = [&](int buf) {
#pragma unroll
    for (int kk = 0; kk < BK / 32; ++kk) {
      const uint32_t w = sW[buf][(wid * 32 + (lane & 31)) * LDW + kk * 2 + (lane >> 5)];
      const i32x4_t wf = unpack16(w);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const i32x4_t af = __builtin_bit_cast(
            i32x4_t, *(const u32x4_t*)&sA[buf][(i * 32 + (lane & 31)) * LDA + kk * 32 + (lane >> 5) * 16]);
        acc[i] = mfma32x32x32_i8(af, wf, acc[i]);
      }
    }
  };

  Regs r0, r1;
  gload(r0, 0);
  gload(r1, 1);
  sstore(r0, 0);
  __syncthreads();
  gload(r0, 2);
  // entering a pair at slice sl: slice sl in LDS buffer 0, sl + 1 in r1, sl + 2 in r0
  int sl = 0;
  for (; sl + 2 <= ns; sl += 2) {
    compute(0);
    sstore(r1, 1);
    __syncthreads();
    gload(r1, sl + 3);
    compute(1);
    sstore(r0, 0);
    __syncthreads();
    gload(r0, sl + 4);
  }
  if (sl < ns) compute(0);  // an odd slice count ends with one more, already in buffer 0

  const Epilogue& e = p.epi;
  const int n = n0 + wid * 32 + (lane & 31);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + i * 32 + mfma32_row(r, lane);
      const bool ok = m < p.M && n < p.N;
      const int accv = acc[i][r];
      if (e.acc_out && ok) e.acc_out[(long)m * p.N + n] = accv;
      const float y = ok ? w2a8_scale(p, m, n, accv) : 0.f;
      if (e.kind == EPI_GEGLU) {
        const float other = __shfl_xor(y, 16, 64);
        if (!(lane & 16) && ok) {
          const float v = gelu_erf(y) * other;
          const long i = (long)m * e.ldo + (n >> 5) * 16 + (lane & 15);
          if (e.out_f32) ((float*)e.out)[i] = v; else ((bf16_t*)e.out)[i] = f2bf(v);
        }
      } else if (ok) {
        if (e.kind == EPI_STORE && e.out) {
          const long i = (long)m * e.ldo + n;
          if (e.out_f32) ((float*)e.out)[i] = y; else ((bf16_t*)e.out)[i] = f2bf(y);
        } else if (e.kind == EPI_RESID) {
          e.resid[(long)m * e.ldr + n] += y;
        }
      }
    }
  }
}

hipError_t gemm_w2a8_scalar(const int8_t* a, int lda, const uint32_t* qp, int M, int N, int K, const Epilogue& epi,
                            float beta_scalar, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (K % 128 || N % 32 || !epi.alpha) return hipErrorInvalidValue;
  W2A8P p{a, lda, qp, M, N, K, (M + 63) / 64, (N + 127) / 128, epi, beta_scalar};
  // 256-wide K slices when they divide K: a weight row's slice is then 64
  // contiguous bytes and the per-slice overhead is spread over twice the MFMAs
  if (K % 256 == 0) hipLaunchKernelGGL(k_gemm_w2a8<256>, dim3(p.nM * p.nN), dim3(256), 0, s, p);
  else hipLaunchKernelGGL(k_gemm_w2a8<128>, dim3(p.nM * p.nN), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t gemm_w2a8(const int8_t* a, int lda, const uint32_t* qp, int M, int N, int K, const Epilogue& epi,
                     hipStream_t s) {
  return gemm_w2a8_scalar(a, lda, qp, M, N, K, epi, 0.f, s);
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
  const Epilogue& e = p.epi;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = m0 + rg * 4 + r;
    if (m >= p.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + cg * 4 + j;
      if (n >= p.N) continue;
      if (e.acc_out) e.acc_out[(long)m * p.N + n] = acc[r][j];
      if (e.out) ((bf16_t*)e.out)[(long)m * e.ldo + n] = f2bf(w2a8_scale(p, m, n, acc[r][j]));
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
