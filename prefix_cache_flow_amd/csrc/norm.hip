// Row kernels: residual update + RMSNorm, and the per-row int8 quantizer of the
// paper's §III-D, Eq. 4.
//
// RMSNorm (the pages do not define the norm; the plainest reading is a pre-norm
// RMSNorm before every sublayer): u = x / sqrt(mean(x^2) + eps) * (1 + w).
// The residual kernel also folds in the split-K partial sums of the projection
// that feeds the residual stream, in a fixed order, so the stream update is
// deterministic.  One 256-thread workgroup per row; a row stays in registers.
//
// Eq. 4: alpha = max(||x||_inf, 1e-5) / 127 in fp32, a = clip(rint(x / alpha),
// -128, 127).  Both divisions are IEEE-rounded fp32 divisions (this library is
// never built with fast-math) and rint rounds ties to even.
#include "common.h"
#include "kernels.h"

namespace vla {

// Element i of a thread's row share: column threadIdx.x + 256 i, or with VEC
// (rows of a multiple of 1024 columns) column 4 (threadIdx.x + 256 (i / 4)) +
// i % 4, so that each thread moves 16-byte vectors.
template <bool VEC>
__device__ __forceinline__ int row_col(int i) {
  return VEC ? (((int)threadIdx.x + (i >> 2) * 256) << 2) + (i & 3) : (int)threadIdx.x + i * 256;
}

template <bool VEC = false>
__device__ __forceinline__ void quantize_store(const float* x, int per, int N, int8_t* q, float* alpha_out,
                                               float* red) {
  float am = 0.f;
  for (int i = 0; i < per; ++i) {
    const int n = row_col<VEC>(i);
    if (n < N) am = fmaxf(am, fabsf(x[i]));
  }
  am = block_max<256>(am, red);
  const float alpha = fmaxf(am, 1e-5f) / 127.0f;
  for (int i = 0; i < per; ++i) {
    const int n = row_col<VEC>(i);
    if (n < N) {
      const float c = rintf(x[i] / alpha);
      q[n] = (int8_t)fminf(fmaxf(c, -128.f), 127.f);
    }
  }
  if (threadIdx.x == 0) *alpha_out = alpha;
}

// NS is a compile-time bound on the split count: every load of the row and of
// its partials is issued before any is used (partials past nsplit re-read the
// last one at a valid address and are masked out).  VEC: see row_col.
template <int PER, int NS, bool VEC>
__global__ __launch_bounds__(256) void k_resid_norm(float* h, int ldh, const float* part, int nsplit, int M, int N,
                                                    const float* gain, float eps, void* u, int u_f32, int ldu,
                                                    int8_t* q, float* alpha, int u_frag, Prefetch pf) {
  static_assert(!VEC || PER % 4 == 0, "vector rows");
  __shared__ float red[4];
  if (prefetch_layer(pf)) return;  // extra workgroups: warm later kernels' weights
  const int m = blockIdx.x;
  constexpr int G = VEC ? 4 : 1;  // consecutive columns per access
  float x[PER];
  float pv[NS > 0 ? NS : 1][PER];
  float ss = 0.f;
  auto load = [&](const float* row, float* dst) {
#pragma unroll
    for (int i = 0; i < PER; i += G) {
      if (VEC) {
        const f32x4_t v = *(const f32x4_t*)(row + row_col<true>(i));
#pragma unroll
        for (int j = 0; j < 4; ++j) dst[i + j] = v[j];
      } else {
        dst[i] = row[min(row_col<false>(i), N - 1)];
      }
    }
  };
  // the gain is requested with the row and its partials: after the block
  // reduction's barrier its loads would be a second memory round trip
  float gk[PER];
#pragma unroll
  for (int i = 0; i < PER; i += G) {
    if (VEC) {
      const f32x4_t gv = *(const f32x4_t*)(gain + row_col<true>(i));
#pragma unroll
      for (int j = 0; j < 4; ++j) gk[i + j] = 1.0f + gv[j];
    } else {
      gk[i] = 1.0f + gain[min(row_col<false>(i), N - 1)];
    }
  }
  load(h + (long)m * ldh, x);
#pragma unroll
  for (int s = 0; s < NS; ++s) load(part + ((long)min(s, nsplit - 1) * M + m) * N, pv[s]);
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int i = 0; i < PER; ++i) x[i] += s < nsplit ? pv[s][i] : 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (row_col<VEC>(i) >= N) x[i] = 0.f;
    ss = fmaf(x[i], x[i], ss);
  }
  if (NS > 0) {
#pragma unroll
    for (int i = 0; i < PER; i += G) {
      const int n = row_col<VEC>(i);
      if (VEC) *(f32x4_t*)(h + (long)m * ldh + n) = f32x4_t{x[i], x[i + 1], x[i + 2], x[i + 3]};
      else if (n < N) h[(long)m * ldh + n] = x[i];
    }
  }
  ss = block_sum<256>(ss, red);
  const float r = 1.0f / sqrtf(ss / (float)N + eps);
#pragma unroll
  for (int i = 0; i < PER; ++i) x[i] = x[i] * r * gk[i];
  if (u) {
#pragma unroll
    for (int i = 0; i < PER; i += G) {
      const int n = row_col<VEC>(i);
      if (VEC) {
        if (u_f32) {
          *(f32x4_t*)((float*)u + (long)m * ldu + n) = f32x4_t{x[i], x[i + 1], x[i + 2], x[i + 3]};
        } else {
          const long o = u_frag ? frag_idx(m, n, N) : (long)m * ldu + n;
          *(u32x2_t*)((bf16_t*)u + o) = u32x2_t{pack_bf2(x[i], x[i + 1]), pack_bf2(x[i + 2], x[i + 3])};
        }
      } else if (n < N) {
        if (u_f32) ((float*)u)[(long)m * ldu + n] = x[i];
        else ((bf16_t*)u)[u_frag ? frag_idx(m, n, N) : (long)m * ldu + n] = f2bf(x[i]);
      }
    }
  }
  if (q) quantize_store<VEC>(x, PER, N, q + (long)m * N, alpha + m, red);
}

template <int PER, bool VEC>
static void launch_rn(int nsplit, hipStream_t s, float* h, int ldh, const float* part, int M, int N,
                      const float* gain, float eps, void* u_out, int u_f32, int ldu, int8_t* q_out, float* alpha_out,
                      int u_frag, const Prefetch& pf) {
#define VLA_RN(NS)                                                                                                  \
  hipLaunchKernelGGL((k_resid_norm<PER, NS, VEC>), dim3(M, 1, prefetch_depth(M, pf.blocks)), dim3(256), 0, s, h, ldh, part, nsplit, M, N, \
                     gain, eps, u_out, u_f32, ldu, q_out, alpha_out, u_frag, pf)
  if (nsplit <= 0) VLA_RN(0);
  else if (nsplit <= 1) VLA_RN(1);
  else if (nsplit <= 4) VLA_RN(4);
  else if (nsplit <= 8) VLA_RN(8);
  else VLA_RN(16);
#undef VLA_RN
}

hipError_t resid_norm(float* h, int ldh, const float* part, int nsplit, int M, int N, const float* gain, float eps,
                      void* u_out, int u_f32, int ldu, int8_t* q_out, float* alpha_out, hipStream_t s, int u_frag,
                      const Prefetch* prefetch) {
  const Prefetch pf = prefetch ? *prefetch : Prefetch{};
  if (pf.blocks < 0 || pf.blocks > 1024 || (pf.blocks && !pf.sink)) return hipErrorInvalidValue;
  if (u_frag && (u_f32 || N % 32)) return hipErrorInvalidValue;
  if (M <= 0) return hipSuccess;
  if (nsplit > 16) return hipErrorInvalidValue;
  const int per = (N + 255) / 256;
  // 16-byte row accesses for rows of a multiple of 1024 columns with aligned strides
  const bool vec = N % 1024 == 0 && ldh % 4 == 0 && (!u_out || ldu % 4 == 0);
#define VLA_RNP(P)                                                                                                \
  (vec ? launch_rn<P, true>(nsplit, s, h, ldh, part, M, N, gain, eps, u_out, u_f32, ldu, q_out, alpha_out, u_frag, pf) \
       : launch_rn<P, false>(nsplit, s, h, ldh, part, M, N, gain, eps, u_out, u_f32, ldu, q_out, alpha_out, u_frag, pf))
  if (per <= 1) launch_rn<1, false>(nsplit, s, h, ldh, part, M, N, gain, eps, u_out, u_f32, ldu, q_out, alpha_out, u_frag, pf);
  else if (per <= 2) launch_rn<2, false>(nsplit, s, h, ldh, part, M, N, gain, eps, u_out, u_f32, ldu, q_out, alpha_out, u_frag, pf);
  else if (per <= 4) VLA_RNP(4);
  else if (per <= 8) VLA_RNP(8);
  else if (per <= 12) VLA_RNP(12);
  else if (per <= 16) VLA_RNP(16);
  else return hipErrorInvalidValue;
#undef VLA_RNP
  return hipGetLastError();
}

template <int PER>
__global__ __launch_bounds__(256) void k_quantize(const float* x, int ldx, int K, int8_t* a, float* alpha) {
  __shared__ float red[4];
  const int m = blockIdx.x;
  float v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int n = threadIdx.x + i * 256;
    v[i] = x[(long)m * ldx + min(n, K - 1)];  // entries past K are never used
  }
  quantize_store(v, PER, K, a + (long)m * K, alpha + m, red);
}

// Rows longer than 16 * 256 elements go through a two-pass loop over global memory.
__global__ __launch_bounds__(256) void k_quantize_long(const float* x, int ldx, int K, int8_t* a, float* alpha) {
  __shared__ float red[4];
  const int m = blockIdx.x;
  const float* row = x + (long)m * ldx;
  float am = 0.f;
  for (int n = threadIdx.x; n < K; n += 256) am = fmaxf(am, fabsf(row[n]));
  am = block_max<256>(am, red);
  const float al = fmaxf(am, 1e-5f) / 127.0f;
  for (int n = threadIdx.x; n < K; n += 256) {
    const float c = rintf(row[n] / al);
    a[(long)m * K + n] = (int8_t)fminf(fmaxf(c, -128.f), 127.f);
  }
  if (threadIdx.x == 0) alpha[m] = al;
}

hipError_t quantize_rows(const float* x, int ldx, int M, int K, int8_t* a, float* alpha, hipStream_t s) {
  if (M <= 0 || K <= 0) return hipSuccess;
  const int per = (K + 255) / 256;
#define VLA_Q(P) hipLaunchKernelGGL(k_quantize<P>, dim3(M), dim3(256), 0, s, x, ldx, K, a, alpha)
  if (per <= 1) VLA_Q(1);
  else if (per <= 4) VLA_Q(4);
  else if (per <= 8) VLA_Q(8);
  else if (per <= 16) VLA_Q(16);
  else if (per <= 28) VLA_Q(28);
  else hipLaunchKernelGGL(k_quantize_long, dim3(M), dim3(256), 0, s, x, ldx, K, a, alpha);
#undef VLA_Q
  return hipGetLastError();
}

}  // namespace vla
