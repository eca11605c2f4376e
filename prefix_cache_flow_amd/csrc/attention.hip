// Softmax attention of the paper's §III-B, Eq. 2, with M = 0 everywhere: the
// prefix is bidirectional (every token sees every other), the expert's
// self-attention covers all chunk tokens, and its cross-attention all cached
// prefix tokens.  Query head j reads key/value head floor(j * Hkv / Hq).
//
// attention_bf16 (MFMA, flash-style).  Each wave owns 32 queries of one head and
// streams the keys in tiles of 32 through LDS, keeping a running max and sum per
// query (online softmax in fp32).  The scores are formed transposed,
// S^T = K Q^T, so every lane holds the 32 key scores of *its* query across its
// accumulator registers: the softmax reductions stay inside a lane pair, and the
// rescaling of the output is one multiply per register.  The output is also
// accumulated transposed, O^T += V^T P^T, with P^T taken straight from the score
// registers (rounded to bf16) and V staged transposed in LDS.  All waves of a
// workgroup share one key/value head, so a K/V tile in LDS serves up to 8 query
// heads (grouped-query attention) or 4 query blocks of one head.
//
// attention_f32: one thread per query row and head, online softmax in fp32
// (the fp32 workload's small shapes).
#include "common.h"
#include "kernels.h"

namespace vla {

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void k_attn_bf16(AttnArgs a, int wgs_per_kvh) {
  constexpr int LDK = D + 8;   // K tile row stride (bf16 elements)
  constexpr int LDV = 32 + 8;  // transposed V tile row stride
  constexpr int NT = 64 * NW;
  __shared__ __attribute__((aligned(16))) uint16_t sK[32 * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t sVt[D * LDV];

  const int QH = a.Hq / a.Hkv;
  const int nQB = (a.Nq + 31) / 32;
  const int items = QH * nQB;
  int bid = blockIdx.x;
  const int b = bid / (a.Hkv * wgs_per_kvh);
  bid -= b * a.Hkv * wgs_per_kvh;
  const int g = bid / wgs_per_kvh;
  const int chunk = bid - g * wgs_per_kvh;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int item = chunk * NW + wid;
  const bool active = item < items;
  const int j = g * QH + (active ? item % QH : 0);
  const int q0 = (active ? item / QH : 0) * 32;
  const int myq = q0 + (lane & 31);
  const bool qvalid = active && myq < a.Nq;
  const int grp = lane >> 5;

  const bf16_t* Q = (const bf16_t*)a.q + b * a.q_bs + j * a.q_hs;
  const bf16_t* K = (const bf16_t*)a.k + b * a.k_bs + g * a.k_hs;
  const bf16_t* V = (const bf16_t*)a.v + b * a.v_bs + g * a.v_hs;

  u32x4_t qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
    qf[s] = qvalid ? *(const u32x4_t*)(Q + (long)myq * a.q_rs + s * 16 + grp * 8) : u32x4_t{0, 0, 0, 0};

  f32x16_t o[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[t][e] = 0.f;
  float mrun = -INFINITY, lrun = 0.f;
  const float sl2 = 1.4426950408889634f / sqrtf((float)D);

  for (int kt = 0; kt < a.Nk; kt += 32) {
    __syncthreads();
    for (int v = threadIdx.x; v < 32 * D / 8; v += NT) {
      const int r = v / (D / 8), c = (v % (D / 8)) * 8;
      const bool ok = kt + r < a.Nk;
      const u32x4_t kv = ok ? *(const u32x4_t*)(K + (long)(kt + r) * a.k_rs + c) : u32x4_t{0, 0, 0, 0};
      *(u32x4_t*)&sK[r * LDK + c] = kv;
      const u32x4_t vv = ok ? *(const u32x4_t*)(V + (long)(kt + r) * a.v_rs + c) : u32x4_t{0, 0, 0, 0};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        sVt[(c + 2 * t) * LDV + r] = (uint16_t)(vv[t] & 0xffffu);
        sVt[(c + 2 * t + 1) * LDV + r] = (uint16_t)(vv[t] >> 16);
      }
    }
    __syncthreads();
    if (!active) continue;

    f32x16_t sacc;
#pragma unroll
    for (int e = 0; e < 16; ++e) sacc[e] = 0.f;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const bf16x8_t kf = as_bf16x8(*(const u32x4_t*)&sK[(lane & 31) * LDK + s * 16 + grp * 8]);
      sacc = mfma32x32x16(kf, as_bf16x8(qf[s]), sacc);
    }
    float mt = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = kt + mfma32_row(e, lane);
      const float x = key < a.Nk ? sacc[e] * sl2 : -INFINITY;
      sacc[e] = x;
      mt = fmaxf(mt, x);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float mnew = fmaxf(mrun, mt);
    const float alpha = exp2f(mrun - mnew);
    float ls = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float pe = exp2f(sacc[e] - mnew);
      sacc[e] = pe;
      ls += pe;
    }
    ls += __shfl_xor(ls, 32, 64);
    lrun = lrun * alpha + ls;
    mrun = mnew;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[t][e] *= alpha;

#pragma unroll
    for (int c = 0; c < 2; ++c) {
      u32x4_t pw;
#pragma unroll
      for (int t = 0; t < 4; ++t) pw[t] = pack_bf2(sacc[8 * c + 2 * t], sacc[8 * c + 2 * t + 1]);
      const bf16x8_t pf = as_bf16x8(pw);
#pragma unroll
      for (int t = 0; t < D / 32; ++t) {
        const uint16_t* row = &sVt[(t * 32 + (lane & 31)) * LDV + 16 * c + grp * 4];
        const u32x2_t lo = *(const u32x2_t*)row;
        const u32x2_t hi = *(const u32x2_t*)(row + 8);
        const u32x4_t vw = {lo[0], lo[1], hi[0], hi[1]};
        o[t] = mfma32x32x16(as_bf16x8(vw), pf, o[t]);
      }
    }
  }

  if (qvalid) {
    const float inv = 1.0f / lrun;
    const long base = b * a.o_bs + (long)myq * a.o_rs + (long)j * D;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int d = t * 32 + mfma32_row(e, lane);
        const float val = o[t][e] * inv;
        if (a.o_f32) ((float*)a.o)[base + d] = val; else ((bf16_t*)a.o)[base + d] = f2bf(val);
      }
  }
}

template <int D, int NW>
static hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t s) {
  const int QH = a.Hq / a.Hkv;
  const int items = QH * ((a.Nq + 31) / 32);
  const int wgs = (items + NW - 1) / NW;
  dim3 grid(a.B * a.Hkv * wgs);
  hipLaunchKernelGGL((k_attn_bf16<D, NW>), grid, dim3(64 * NW), 0, s, a, wgs);
  return hipGetLastError();
}

hipError_t attention_bf16(const AttnArgs& a, hipStream_t s) {
  if (a.B <= 0 || a.Nq <= 0 || a.Nk <= 0) return hipSuccess;
  if (a.Hq % a.Hkv) return hipErrorInvalidValue;
  const bool gqa8 = (a.Hq / a.Hkv) % 8 == 0;
  switch (a.hd) {
    case 64: return gqa8 ? launch_attn_bf16<64, 8>(a, s) : launch_attn_bf16<64, 4>(a, s);
    case 128: return gqa8 ? launch_attn_bf16<128, 8>(a, s) : launch_attn_bf16<128, 4>(a, s);
    case 256: return gqa8 ? launch_attn_bf16<256, 8>(a, s) : launch_attn_bf16<256, 4>(a, s);
    default: return hipErrorInvalidValue;
  }
}

// ------------------------------------------------------------------ fp32
template <int D>
__global__ __launch_bounds__(64) void k_attn_f32(AttnArgs a) {
  const int i = blockIdx.x * 64 + threadIdx.x;
  const int j = blockIdx.y, b = blockIdx.z;
  if (i >= a.Nq) return;
  const int g = j * a.Hkv / a.Hq;
  const float* q = (const float*)a.q + b * a.q_bs + j * a.q_hs + (long)i * a.q_rs;
  const float* K = (const float*)a.k + b * a.k_bs + g * a.k_hs;
  const float* V = (const float*)a.v + b * a.v_bs + g * a.v_hs;
  float qv[D], o[D];
  const float sc = 1.0f / sqrtf((float)D);
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qv[d] = q[d] * sc;
    o[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int t = 0; t < a.Nk; ++t) {
    const float* kr = K + (long)t * a.k_rs;
    float s = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) s = fmaf(qv[d], kr[d], s);
    const float mn = fmaxf(m, s);
    const float al = expf(m - mn), p = expf(s - mn);
    l = l * al + p;
    const float* vr = V + (long)t * a.v_rs;
#pragma unroll
    for (int d = 0; d < D; ++d) o[d] = fmaf(p, vr[d], o[d] * al);
    m = mn;
  }
  float* out = (float*)a.o + b * a.o_bs + (long)i * a.o_rs + (long)j * D;
  const float inv = 1.0f / l;
#pragma unroll
  for (int d = 0; d < D; ++d) out[d] = o[d] * inv;
}

hipError_t attention_f32(const AttnArgs& a, hipStream_t s) {
  if (a.B <= 0 || a.Nq <= 0 || a.Nk <= 0) return hipSuccess;
  if (a.Hq % a.Hkv || !a.o_f32) return hipErrorInvalidValue;
  dim3 grid((a.Nq + 63) / 64, a.Hq, a.B);
  switch (a.hd) {
    case 32: hipLaunchKernelGGL(k_attn_f32<32>, grid, dim3(64), 0, s, a); break;
    case 64: hipLaunchKernelGGL(k_attn_f32<64>, grid, dim3(64), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace vla
