// Row kernels of the action expert's solver loop: the chunk-token embedding
// with the solver time, and the velocity head fused with the Euler update of
// the paper's §III-A, Eq. 1: X^{k+1} = X^k + (tau_{k+1} - tau_k) v(X^k, tau_k).
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

// Head of step k fused with the embedding of step k + 1, one 256-thread
// workgroup per chunk row (both are row-local): final RMSNorm, W_out and the
// Euler update, then the new row through W_in plus phi(tau_{k+1}) and the first
// layer's RMSNorm.  Either part can be switched off (first and last step).  In
// their fast forms (bf16 weights and d_e <= 1024, d_a <= 32; the head also
// needs d_e % 64 == 0, the embedding d_a % 8 == 0) every weight vector is
// requested before the row itself is read, so the kernel is one memory round
// trip.  Each part's form depends on the shapes alone.
template <bool WF32, bool FH, bool FE>
__global__ __launch_bounds__(256) void k_step_rows(StepRows a) {
  __shared__ float red[4];
  __shared__ float us[4096];
  __shared__ float xs[256];
  if (prefetch_layer(a.pf)) return;  // extra workgroups: warm the next kernel's weights
  const int m = blockIdx.x;
  const int tid = threadIdx.x;
  const bool head = a.k_head >= 0, emb = a.k_embed >= 0;
  constexpr int G = 8;  // threads per head output
  const int part = tid % G, ao = tid / G;
  // ---- every global operand first (fast forms): weights, the row, both gains,
  // the schedule entries and the action values this thread updates (read after
  // a barrier, each would be one more memory round trip)
  constexpr int PER = 4;  // row elements per thread when d_e <= 1024
  u32x4_t wo[16], wi[16];
  float er[PER], gf[PER], g1[PER];
  const float dt = head ? a.sched[a.k_head + 1] - a.sched[a.k_head] : 0.f;
  const float tau = emb ? a.sched[a.k_embed] : 0.f;
  const bool xown = FH && head && part == 0 && ao < a.d_a;
  const float x0 = xown ? a.X[(long)m * a.d_a + ao] : 0.f;
  if (FH && head) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int n = min(tid + i * 256, a.d_e - 1);
      er[i] = a.E[(long)m * a.d_e + n];
      gf[i] = a.gain_f[n];
    }
  }
  if (FE && emb) {
#pragma unroll
    for (int i = 0; i < PER; ++i) g1[i] = a.gain_1[min(tid + i * 256, a.d_e - 1)];
  }
  {
    if (FH && head) {
      const int sl = a.d_e / G;  // slice of a W_out row per thread, multiple of 8
      const bf16_t* wr = (const bf16_t*)a.w_out + (long)min(ao, a.d_a - 1) * a.d_e + part * sl;
#pragma unroll
      for (int t = 0; t < 16; ++t) wo[t] = *(const u32x4_t*)(wr + min(t * 8, sl - 8));
    }
    if (FE && emb) {
      const int dv = a.d_a / 8;  // vectors per W_in row
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const int i = t / 4, v = t % 4;  // output tid + 256 i, vector v of its row
        const int n = min(tid + i * 256, a.d_e - 1);
        wi[t] = *(const u32x4_t*)((const bf16_t*)a.w_in + (long)n * a.d_a + min(v, dv - 1) * 8);
      }
    }
  }
  // ---- head: v = RMS(E; w_ef) W_out^T, X += dt v
  if (head) {
    float ss = 0.f;
    if (FH) {
#pragma unroll
      for (int i = 0; i < PER; ++i) ss = fmaf(er[i], tid + i * 256 < a.d_e ? er[i] : 0.f, ss);
      ss = block_sum<256>(ss, red);
      const float r = 1.0f / sqrtf(ss / (float)a.d_e + a.eps);
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if (tid + i * 256 < a.d_e) us[tid + i * 256] = er[i] * r * (1.0f + gf[i]);
    } else {
      for (int n = tid; n < a.d_e; n += 256) {
        const float v = a.E[(long)m * a.d_e + n];
        us[n] = v;
        ss = fmaf(v, v, ss);
      }
      ss = block_sum<256>(ss, red);
      const float r = 1.0f / sqrtf(ss / (float)a.d_e + a.eps);
      for (int n = tid; n < a.d_e; n += 256) us[n] = us[n] * r * (1.0f + a.gain_f[n]);
    }
    __syncthreads();
    if (FH) {
      const int sl = a.d_e / G;
      float acc = 0.f;
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        if (t * 8 >= sl) break;
        const float* ur = &us[part * sl + t * 8];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          acc = fmaf(ur[2 * h], bf2f((bf16_t)(wo[t][h] & 0xffffu)), acc);
          acc = fmaf(ur[2 * h + 1], bf2f((bf16_t)(wo[t][h] >> 16)), acc);
        }
      }
#pragma unroll
      for (int o = 1; o < G; o <<= 1) acc += __shfl_xor(acc, o, 64);
      if (xown) {
        const float x = x0 + dt * acc;
        a.X[(long)m * a.d_a + ao] = x;
        xs[ao] = x;
      }
    } else {
      for (int o = ao; o < a.d_a; o += 256 / G) {
        float acc = 0.f;
        for (int n = part; n < a.d_e; n += G) acc = fmaf(us[n], ld_w<WF32>(a.w_out, (long)o * a.d_e + n), acc);
#pragma unroll
        for (int q = 1; q < G; q <<= 1) acc += __shfl_xor(acc, q, 64);
        if (part == 0) {
          const float x = a.X[(long)m * a.d_a + o] + dt * acc;
          a.X[(long)m * a.d_a + o] = x;
          xs[o] = x;
        }
      }
    }
  } else if (tid < a.d_a) {
    xs[tid] = a.X[(long)m * a.d_a + tid];
  }
  if (!emb) return;
  __syncthreads();
  // ---- embedding of step k_embed: E = X W_in^T + phi(tau), u = RMS(E; a1)
  const float l2 = 13.287712379549449f;  // log2(10000)
  float ss = 0.f;
  // the embedded row element n = tid + 256 i
  auto emit = [&](int n, float v) {
    // phi: frequency 10000^(-2i/d) on the exponential unit, angle tau * freq <= |tau|
    const float freq = fast_exp2(-l2 * (2.0f * (float)(n >> 1) / (float)a.d_e));
    const float arg = tau * freq;
    v += (n & 1) ? __cosf(arg) : __sinf(arg);
    a.Eout[(long)m * a.d_e + n] = v;
    us[n] = v;
    ss = fmaf(v, v, ss);
  };
  if (FE) {
    const int dv = a.d_a / 8;
#pragma unroll
    for (int i = 0; i < PER; ++i) {  // unrolled: the weight registers are indexed statically
      const int n = tid + i * 256;
      if (n >= a.d_e) break;
      float v = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (q >= dv) break;
        const u32x4_t w = wi[i * 4 + q];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          v = fmaf(xs[q * 8 + 2 * h], bf2f((bf16_t)(w[h] & 0xffffu)), v);
          v = fmaf(xs[q * 8 + 2 * h + 1], bf2f((bf16_t)(w[h] >> 16)), v);
        }
      }
      emit(n, v);
    }
  } else {
    for (int n = tid; n < a.d_e; n += 256) {
      float v = 0.f;
      for (int a0 = 0; a0 < a.d_a; ++a0) v = fmaf(xs[a0], ld_w<WF32>(a.w_in, (long)n * a.d_a + a0), v);
      emit(n, v);
    }
  }
  ss = block_sum<256>(ss, red);
  const float r = 1.0f / sqrtf(ss / (float)a.d_e + a.eps);
  auto put_u = [&](int n, float g) {
    const float un = us[n] * r * (1.0f + g);
    if (a.u_f32) ((float*)a.u)[(long)m * a.d_e + n] = un;
    else ((bf16_t*)a.u)[a.u_frag ? frag_idx(m, n, a.d_e) : (long)m * a.d_e + n] = f2bf(un);
  };
  if (FE) {
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (tid + i * 256 < a.d_e) put_u(tid + i * 256, g1[i]);
  } else {
    for (int n = tid; n < a.d_e; n += 256) put_u(n, a.gain_1[n]);
  }
}

hipError_t step_rows(const StepRows& a, int w_f32, hipStream_t s) {
  if (a.M <= 0 || (a.k_head < 0 && a.k_embed < 0)) return hipSuccess;
  if (a.d_a > 256 || a.d_e > 4096) return hipErrorInvalidValue;
  if (a.k_embed >= 0 && a.u_frag && (a.u_f32 || a.d_e % 32)) return hipErrorInvalidValue;
  if (a.pf.blocks < 0 || a.pf.blocks > 1024 || (a.pf.blocks && !a.pf.sink)) return hipErrorInvalidValue;
  // each part's form depends on the shapes only, so a step computes the same bits fused or alone
  const bool fh = !w_f32 && a.d_e % 64 == 0 && a.d_e <= 1024 && a.d_a <= 32;
  const bool fe = !w_f32 && a.d_a % 8 == 0 && a.d_a <= 32 && a.d_e <= 1024;
  const dim3 grid(a.M, 1, prefetch_depth(a.M, a.pf.blocks));
  if (w_f32) hipLaunchKernelGGL((k_step_rows<true, false, false>), grid, dim3(256), 0, s, a);
  else if (fh && fe) hipLaunchKernelGGL((k_step_rows<false, true, true>), grid, dim3(256), 0, s, a);
  else if (fh) hipLaunchKernelGGL((k_step_rows<false, true, false>), grid, dim3(256), 0, s, a);
  else if (fe) hipLaunchKernelGGL((k_step_rows<false, false, true>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((k_step_rows<false, false, false>), grid, dim3(256), 0, s, a);
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

struct Lengths64 {
  int v[64];
};
__global__ void k_set_lengths(int* dst, Lengths64 l, int n) {
  if ((int)threadIdx.x < n) dst[threadIdx.x] = l.v[threadIdx.x];
}

hipError_t set_lengths(int* dst, const int32_t* len, int B, int N, hipStream_t s) {
  for (int b0 = 0; b0 < B; b0 += 64) {
    Lengths64 l;
    const int n = std::min(64, B - b0);
    for (int i = 0; i < 64; ++i) l.v[i] = i < n ? (len ? len[b0 + i] : N) : 0;
    hipLaunchKernelGGL(k_set_lengths, dim3(1), dim3(64), 0, s, dst + b0, l, n);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// One prefix row of d values per workgroup into the fp32 residual stream: fp32
// copied, bf16 widened (exact); rows past the observation's length (lens, if
// given) become zeros.
template <bool BF16>
__global__ void k_copy_prefix_rows(const void* src, float* dst, int N, int d, const int* lens) {
  const long row = blockIdx.x;
  const int b = (int)(row / N), t = (int)(row % N);
  const bool keep = !lens || t < lens[b];
  for (int i = threadIdx.x; i < d; i += blockDim.x) {
    const float v = BF16 ? bf2f(((const bf16_t*)src)[row * d + i]) : ((const float*)src)[row * d + i];
    dst[row * d + i] = keep ? v : 0.f;
  }
}

hipError_t copy_prefix_rows(const void* src, int src_bf16, float* dst, int B, int N, int d, const int* lens,
                            hipStream_t s) {
  if ((long)B * N <= 0) return hipSuccess;
  if ((long)B * N > 0x7fffffffL) return hipErrorInvalidValue;
  if (src_bf16) hipLaunchKernelGGL(k_copy_prefix_rows<true>, dim3((unsigned)(B * N)), dim3(256), 0, s, src, dst, N, d, lens);
  else hipLaunchKernelGGL(k_copy_prefix_rows<false>, dim3((unsigned)(B * N)), dim3(256), 0, s, src, dst, N, d, lens);
  return hipGetLastError();
}

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

// ------------------------------------------------------------------ absorbed cross attention
// The cross-attention scores of query head j are u Wq_j^T K_g^T and its output
// enters the residual as softmax(.) V_g Wo_j^T (the paper's §III-B: the cached
// K_g and V_g are fixed while the solver runs), so for one observation the
// products Wq_j^T K_g^T and V_g Wo_j^T can be formed once per layer; a solver
// step then needs two products per cross sublayer (scores, and weights times
// Wvo into the residual) instead of query, attention and output kernels.
//
// k_absorb<HD, QK>: one layer, one query head j, 288 keys (18 key blocks) and
// 256 output features (eight waves of 2 row blocks, two per SIMD).  The keys'
// (QK) or values' fragments of every d-step are staged once in LDS and shared
// by the eight waves; each wave requests all its rows of WqT (QK) or Wo (the
// other operand, columns j hd .. j hd + hd - 1) up front, so a workgroup waits
// on memory once.
//   QK: D[k][t] = sum_d WqT[k][j hd + d] K[t][d]: a lane's four results are four
//       consecutive k of output row j Np + t of wqk (one 8-byte store, scaled by
//       sl2 = log2(e) / sqrt(hd)).
//   VO: D[t][n] = sum_d V[t][d] Wo[n][j hd + d]: four consecutive keys of row n,
//       column j Np + t of wvo (padding keys have zero values: zero columns).
constexpr int kAbsXB = 18, kAbsYB = 2;

template <int HD, bool QK>
__global__ __launch_bounds__(512) void k_absorb(AbsorbP p) {
  constexpr int DS = HD / 32, XB = kAbsXB, YB = kAbsYB, NX = DS * XB * 64;
  __shared__ u32x4_t xs[DS * XB][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int tbs = p.Np / 16, tcs = (tbs + XB - 1) / XB, ybs = p.d_e / 16;
  const int j = blockIdx.y / tcs, tc = blockIdx.y % tcs, l = blockIdx.z;
  const int g = j * p.Hkv / p.Hq, qe = p.Hq * HD;
  const int tb0 = tc * XB, yb0 = (blockIdx.x * 8 + w) * YB;
  const u32x4_t* X = (const u32x4_t*)((QK ? p.k + l * p.k_ls : p.v + l * p.v_ls) + (long)g * p.Np * HD);
  const u32x4_t* Y = (const u32x4_t*)(QK ? p.wqT + l * p.wq_ls : p.wo + l * p.wo_ls) + (long)j * DS * 64 + lane;
  // every d-step of this wave's rows requested first, then the shared blocks
  u32x4_t y[DS][YB];
#pragma unroll
  for (int ds = 0; ds < DS; ++ds)
#pragma unroll
    for (int a = 0; a < YB; ++a) y[ds][a] = Y[((long)min(yb0 + a, ybs - 1) * (qe / 32) + ds) * 64];
  // shared operand: blocks tb0 .. tb0 + XB - 1 (clamped), every d-step
#pragma unroll
  for (int r = 0; r < (NX + 511) / 512; ++r) {
    const int i = r * 512 + (int)threadIdx.x;
    if (NX % 512 == 0 || i < NX) {
      const int f = i >> 6, ln = i & 63, xb = f / DS, ds = f - xb * DS;
      xs[ds * XB + xb][ln] = X[((long)min(tb0 + xb, tbs - 1) * DS + ds) * 64 + ln];
    }
  }
  __syncthreads();
  if (yb0 >= ybs) return;
  f32x4_t acc[YB][XB];
#pragma unroll
  for (int a = 0; a < YB; ++a)
#pragma unroll
    for (int i = 0; i < XB; ++i) acc[a][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ds = 0; ds < DS; ++ds)
#pragma unroll
    for (int i = 0; i < XB; ++i) {
      const u32x4_t x = xs[ds * XB + i][lane];
#pragma unroll
      for (int a = 0; a < YB; ++a)
        acc[a][i] = QK ? mfma16x16x32(as_bf16x8(y[ds][a]), as_bf16x8(x), acc[a][i])
                       : mfma16x16x32(as_bf16x8(x), as_bf16x8(y[ds][a]), acc[a][i]);
    }
  const int ns = p.Hq * p.Np;
  uint16_t* out = (QK ? p.wqk : p.wvo) + l * p.out_ls;
#pragma unroll
  for (int a = 0; a < YB; ++a) {
    if (yb0 + a >= ybs) break;
#pragma unroll
    for (int i = 0; i < XB; ++i) {
      if (tb0 + i >= tbs) break;
      if (QK) {
        const int k = (yb0 + a) * 16 + grp * 4, t = (tb0 + i) * 16 + col;
        const u32x2_t pk = {pack_bf2(acc[a][i][0] * p.sl2, acc[a][i][1] * p.sl2),
                            pack_bf2(acc[a][i][2] * p.sl2, acc[a][i][3] * p.sl2)};
        *(u32x2_t*)(out + frag_idx(j * p.Np + t, k, p.d_e)) = pk;
      } else {
        const int t = (tb0 + i) * 16 + grp * 4, n = (yb0 + a) * 16 + col;
        const u32x2_t pk = {pack_bf2(acc[a][i][0], acc[a][i][1]), pack_bf2(acc[a][i][2], acc[a][i][3])};
        *(u32x2_t*)(out + frag_idx(n, j * p.Np + t, ns)) = pk;
      }
    }
  }
}

hipError_t absorb_products(const AbsorbP& p, hipStream_t s) {
  if (p.L <= 0) return hipSuccess;
  if (!p.k || !p.v || !p.wqT || !p.wo || !p.wqk || !p.wvo || p.Hq <= 0 || p.Hkv <= 0 || p.Hq % p.Hkv ||
      p.Np <= 0 || p.Np % 32 || p.d_e <= 0 || p.d_e % 128)
    return hipErrorInvalidValue;
  const int tbs = p.Np / 16, ybs = p.d_e / 16;
  const dim3 grid((ybs + 8 * kAbsYB - 1) / (8 * kAbsYB), p.Hq * ((tbs + kAbsXB - 1) / kAbsXB), p.L);
  switch (p.hd) {
    case 64:
      hipLaunchKernelGGL((k_absorb<64, true>), grid, dim3(512), 0, s, p);
      hipLaunchKernelGGL((k_absorb<64, false>), grid, dim3(512), 0, s, p);
      break;
    case 128:
      hipLaunchKernelGGL((k_absorb<128, true>), grid, dim3(512), 0, s, p);
      hipLaunchKernelGGL((k_absorb<128, false>), grid, dim3(512), 0, s, p);
      break;
    case 256:
      hipLaunchKernelGGL((k_absorb<256, true>), grid, dim3(512), 0, s, p);
      hipLaunchKernelGGL((k_absorb<256, false>), grid, dim3(512), 0, s, p);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace vla
