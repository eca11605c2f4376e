// Small row kernels of the action expert: the chunk-token embedding with the
// solver time, and the velocity head fused with the Euler update of the
// paper's §III-A, Eq. 1: X^{k+1} = X^k + (tau_{k+1} - tau_k) v(X^k, tau_k).
//
// The time embedding is not defined on the pages; the plainest reading of a
// sinusoidal embedding of tau is used: phi_{2i} = sin(tau / 10000^(2i/d)),
// phi_{2i+1} = cos(tau / 10000^(2i/d)), added to every chunk token after the
// input projection.  tau_k and tau_{k+1} are read from a device copy of the
// schedule, so one captured graph serves any schedule of the same length.
#include "common.h"
#include "kernels.h"

namespace vla {

template <bool WF32>
__device__ __forceinline__ float ld_w(const void* w, long i) {
  if (WF32) return ((const float*)w)[i];
  return bf2f(((const bf16_t*)w)[i]);
}

// One 256-thread workgroup per chunk row m; d_e <= 4096, d_a <= 256.  The
// row's d_a inputs sit in LDS; each thread loads its weight rows for all of
// its outputs before using any (clamped indices, masked products).
template <bool WF32>
__global__ __launch_bounds__(256) void k_embed(const float* X, int d_a, const void* w_in, int d_e, const float* sched,
                                               int k, float* E, const float* gain, float eps, void* u, int u_f32,
                                               int u_frag, int M, Prefetch pf) {
  __shared__ float xs[256];
  __shared__ float es[4096];
  if ((int)blockIdx.x >= M) {  // extra workgroups: warm the next kernel's weights
    prefetch_share(pf, blockIdx.x - M, gridDim.x - M);
    return;
  }
  __shared__ float red[4];
  const int m = blockIdx.x;
  if (threadIdx.x < d_a) xs[threadIdx.x] = X[(long)m * d_a + threadIdx.x];
  __syncthreads();
  const float tau = sched[k];
  const float l2 = 13.287712379549449f;  // log2(10000)
  float ss = 0.f;
  for (int n = threadIdx.x; n < d_e; n += 256) {
    float v = 0.f;
    for (int a0 = 0; a0 < d_a; a0 += 8) {
      float wv[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) wv[t] = ld_w<WF32>(w_in, (long)n * d_a + min(a0 + t, d_a - 1));
#pragma unroll
      for (int t = 0; t < 8; ++t) v = fmaf(a0 + t < d_a ? xs[a0 + t] : 0.f, wv[t], v);
    }
    // phi: frequency 10000^(-2i/d) on the exponential unit, angle tau * freq <= |tau|
    const float freq = fast_exp2(-l2 * (2.0f * (float)(n >> 1) / (float)d_e));
    const float arg = tau * freq;
    v += (n & 1) ? __cosf(arg) : __sinf(arg);
    E[(long)m * d_e + n] = v;
    es[n] = v;
    ss = fmaf(v, v, ss);
  }
  ss = block_sum<256>(ss, red);
  const float r = 1.0f / sqrtf(ss / (float)d_e + eps);
  for (int n = threadIdx.x; n < d_e; n += 256) {
    const float un = es[n] * r * (1.0f + gain[n]);
    if (u_f32) ((float*)u)[(long)m * d_e + n] = un;
    else ((bf16_t*)u)[u_frag ? frag_idx(m, n, d_e) : (long)m * d_e + n] = f2bf(un);
  }
}

hipError_t expert_embed(const float* X, int M, int d_a, const void* w_in, int w_f32, int d_e, const float* sched,
                        int k, float* E, const float* gain, float eps, void* u, int u_f32, hipStream_t s, int u_frag,
                        const Prefetch* prefetch) {
  if (M <= 0) return hipSuccess;
  if (d_a > 256 || d_e > 4096) return hipErrorInvalidValue;
  if (u_frag && (u_f32 || d_e % 32 || M > 64)) return hipErrorInvalidValue;
  const Prefetch pf = prefetch ? *prefetch : Prefetch{};
  if (pf.blocks < 0 || pf.blocks > 1024 || (pf.blocks && !pf.sink)) return hipErrorInvalidValue;
  if (w_f32)
    hipLaunchKernelGGL(k_embed<true>, dim3(M + pf.blocks), dim3(256), 0, s, X, d_a, w_in, d_e, sched, k, E, gain, eps,
                       u, u_f32, u_frag, M, pf);
  else
    hipLaunchKernelGGL(k_embed<false>, dim3(M + pf.blocks), dim3(256), 0, s, X, d_a, w_in, d_e, sched, k, E, gain,
                       eps, u, u_f32, u_frag, M, pf);
  return hipGetLastError();
}

// One 256-thread workgroup per chunk row: final RMSNorm, W_out, Euler update.
// The normalized row goes to LDS; then G = 8 threads share each output: thread
// t takes output t / 8 (and every 32nd after it) and the t % 8-th slice of the
// row, loads that slice of the weight row before using it, and the eight
// partial dot products are summed with lane exchanges in a fixed order.
template <bool WF32>
__global__ __launch_bounds__(256) void k_head(const float* E, int d_e, const float* gain, float eps, const void* w_out,
                                              int d_a, const float* sched, int k, float* X) {
  __shared__ float red[4];
  __shared__ float us[4096];
  const int m = blockIdx.x;
  float ss = 0.f;
  for (int n = threadIdx.x; n < d_e; n += 256) {
    const float v = E[(long)m * d_e + n];
    us[n] = v;
    ss = fmaf(v, v, ss);
  }
  ss = block_sum<256>(ss, red);
  const float r = 1.0f / sqrtf(ss / (float)d_e + eps);
  for (int n = threadIdx.x; n < d_e; n += 256) us[n] = us[n] * r * (1.0f + gain[n]);
  __syncthreads();
  const float dt = sched[k + 1] - sched[k];
  constexpr int G = 8;
  const int slice = d_e / G;  // d_e % 64 == 0 for bf16 weights (8-element vectors)
  const int part = threadIdx.x % G;
  for (int a = threadIdx.x / G; a < d_a; a += 256 / G) {
    float acc = 0.f;
    if (WF32) {
      for (int n = part; n < d_e; n += G) acc = fmaf(us[n], ld_w<true>(w_out, (long)a * d_e + n), acc);
    } else {
      const bf16_t* wr = (const bf16_t*)w_out + (long)a * d_e + part * slice;
      for (int c = 0; c < slice; c += 128) {  // 16 vectors of 8 weights in flight at once
        u32x4_t wv[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) wv[t] = *(const u32x4_t*)(wr + min(c + t * 8, slice - 8));
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          if (c + t * 8 >= slice) break;
          const float* ur = &us[part * slice + c + t * 8];
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            acc = fmaf(ur[2 * h], bf2f((bf16_t)(wv[t][h] & 0xffffu)), acc);
            acc = fmaf(ur[2 * h + 1], bf2f((bf16_t)(wv[t][h] >> 16)), acc);
          }
        }
      }
    }
#pragma unroll
    for (int o = 1; o < G; o <<= 1) acc += __shfl_xor(acc, o, 64);
    if (part == 0) X[(long)m * d_a + a] += dt * acc;
  }
}

hipError_t expert_head(const float* E, int M, int d_e, const float* gain, float eps, const void* w_out, int w_f32,
                       int d_a, const float* sched, int k, float* X, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (d_e > 4096) return hipErrorInvalidValue;
  if (w_f32)
    hipLaunchKernelGGL(k_head<true>, dim3(M), dim3(256), 0, s, E, d_e, gain, eps, w_out, d_a, sched, k, X);
  else
    hipLaunchKernelGGL(k_head<false>, dim3(M), dim3(256), 0, s, E, d_e, gain, eps, w_out, d_a, sched, k, X);
  return hipGetLastError();
}

__global__ void k_copy_out(const float* src, void* dst, long n, int out_bf16) {
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) {
    if (out_bf16) ((bf16_t*)dst)[i] = f2bf(src[i]); else ((float*)dst)[i] = src[i];
  }
}

hipError_t copy_out(const float* src, void* dst, long n, int out_bf16, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int blocks = (int)std::min<long>((n + 255) / 256, 1024);
  hipLaunchKernelGGL(k_copy_out, dim3(blocks), dim3(256), 0, s, src, dst, n, out_bf16);
  return hipGetLastError();
}

hipError_t copy_f32(const float* src, float* dst, long n, hipStream_t s) { return copy_out(src, dst, n, 0, s); }

__global__ void k_f32_to_bf16(const float* src, uint16_t* dst, long n) {
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x)
    dst[i] = f2bf(src[i]);
}

hipError_t f32_to_bf16(const float* src, uint16_t* dst, long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int blocks = (int)std::min<long>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(k_f32_to_bf16, dim3(blocks), dim3(256), 0, s, src, dst, n);
  return hipGetLastError();
}

// zero the last `tail` 16-bit elements of each of `nblk` blocks of `blk` elements
__global__ void k_zero_tails(uint16_t* base, long blk, int tail) {
  uint16_t* p = base + (long)blockIdx.x * blk + (blk - tail);
  for (int i = threadIdx.x * 8; i < tail; i += blockDim.x * 8) *(u32x4_t*)(p + i) = u32x4_t{0u, 0u, 0u, 0u};
}

hipError_t zero_tails(void* base, long nblk, long blk, int tail, hipStream_t s) {
  if (nblk <= 0 || tail <= 0) return hipSuccess;
  if (tail % 8 || blk % 8 || tail > blk || nblk > 0x7fffffffL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_zero_tails, dim3((unsigned)nblk), dim3(256), 0, s, (uint16_t*)base, blk, tail);
  return hipGetLastError();
}

}  // namespace vla
