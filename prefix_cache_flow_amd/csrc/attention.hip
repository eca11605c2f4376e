// Softmax attention of the paper's §III-B, Eq. 2, with M = 0 everywhere: the
// prefix is bidirectional (every token sees every other), the expert's
// self-attention covers all chunk tokens, and its cross-attention all cached
// prefix tokens.  Query head j reads key/value head floor(j * Hkv / Hq).
//
// attention_bf16 (MFMA, flash-style).  A workgroup of four waves owns 16
// queries of one head; the four waves split the keys into four ranges and
// each streams its range in tiles of 32 keys through its own slice of LDS,
// keeping a running max and sum per query (online softmax in fp32).  The
// scores are formed transposed on the 16x16x32 bf16 MFMA, S^T = K Q^T, so every
// lane holds the scores of *its* query in registers: the softmax reductions
// are two lane exchanges, and rescaling the output is one multiply per
// register.  The output is accumulated transposed too, O^T += V^T P^T, with
// P^T taken straight from the score registers (rounded to bf16) in a key
// order that the transposed V tile in LDS reproduces.  At the end the four
// partial results are merged through LDS in a fixed order.  Splitting keys
// inside the workgroup gives (queries / 16) x heads workgroups, enough to
// spread even a 50-token chunk over the chip.
//
// attention_f32: one thread per query row and head, online softmax in fp32
// (the fp32 workload's small shapes).
#include "common.h"
#include "kernels.h"

namespace vla {

template <int D>
__global__ __launch_bounds__(256) void k_attn16(AttnArgs a) {
  constexpr int LDK = D + 8;   // K tile row stride (bf16)
  constexpr int LDV = 36;      // transposed V tile row stride: 32 keys + 4 (conflict-free u32 writes)
  constexpr int WAVE_LDS = 32 * LDK + D * LDV;
  constexpr int LDO = D + 4;   // merge buffer row stride (floats)
  static_assert(2 * WAVE_LDS * 4 >= 4 * (128 + 64 * LDO), "merge buffer must fit in the staging area");
  __shared__ __attribute__((aligned(16))) uint16_t lds[4 * WAVE_LDS];

  const int j = blockIdx.x % a.Hq, qb = blockIdx.x / a.Hq, b = blockIdx.y;
  const int g = j * a.Hkv / a.Hq;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int myq = qb * 16 + col;

  const bf16_t* Q = (const bf16_t*)a.q + b * a.q_bs + j * a.q_hs;
  const bf16_t* K = (const bf16_t*)a.k + b * a.k_bs + g * a.k_hs;
  const bf16_t* V = (const bf16_t*)a.v + b * a.v_bs + g * a.v_hs;

  // Rows past the end are clamped to the last valid row instead of branching
  // around the load (a branch per load serialises the memory accesses): a
  // clamped query is never stored, a clamped key gets a score of -inf and so a
  // weight of exactly 0 on its (finite) value row.
  const int qrow = min(myq, a.Nq - 1);
  u32x4_t qf[D / 32];
#pragma unroll
  for (int s = 0; s < D / 32; ++s) qf[s] = *(const u32x4_t*)(Q + (long)qrow * a.q_rs + s * 32 + grp * 8);

  f32x4_t o[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) o[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float mrun = -INFINITY, lrun = 0.f;
  const float sl2 = 1.4426950408889634f / sqrtf((float)D);

  uint16_t* sK = lds + w * WAVE_LDS;
  uint16_t* sVt = sK + 32 * LDK;
  const int T = (a.Nk + 31) / 32;
  const int t0 = (w * T) / 4, t1 = ((w + 1) * T) / 4;
  // one tile of K ([32][D], D/16 vectors per lane) and V (keys 2p, 2p+1 of 8 d per vector) in registers
  u32x4_t kr[D / 16], vr0[D / 32], vr1[D / 32];
  const int p = lane & 15, dg = lane >> 4;
  auto fetch = [&](int kt) {
#pragma unroll
    for (int i = 0; i < D / 16; ++i) {
      const int v = lane + i * 64, r = v / (D / 8), c = (v % (D / 8)) * 8;
      kr[i] = *(const u32x4_t*)(K + (long)min(kt + r, a.Nk - 1) * a.k_rs + c);
    }
    const long r0 = min(kt + 2 * p, a.Nk - 1), r1 = min(kt + 2 * p + 1, a.Nk - 1);
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
      vr0[i] = *(const u32x4_t*)(V + r0 * a.v_rs + i * 32 + dg * 8);
      vr1[i] = *(const u32x4_t*)(V + r1 * a.v_rs + i * 32 + dg * 8);
    }
  };
  if (t0 < t1) fetch(t0 * 32);
  for (int t = t0; t < t1; ++t) {
    const int kt = t * 32;
    // K tile row-major; V tile transposed [D][32] written as 32-bit key pairs
#pragma unroll
    for (int i = 0; i < D / 16; ++i) {
      const int v = lane + i * 64, r = v / (D / 8), c = (v % (D / 8)) * 8;
      *(u32x4_t*)&sK[r * LDK + c] = kr[i];
    }
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
      const int d0 = i * 32 + dg * 8;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const uint32_t lo = (vr0[i][h] & 0xffffu) | (vr1[i][h] << 16);
        const uint32_t hi = (vr0[i][h] >> 16) | (vr1[i][h] & 0xffff0000u);
        *(uint32_t*)&sVt[(d0 + 2 * h) * LDV + 2 * p] = lo;
        *(uint32_t*)&sVt[(d0 + 2 * h + 1) * LDV + 2 * p] = hi;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (t + 1 < t1) fetch(kt + 32);  // next tile in flight during this tile's math

    // S^T = K Q^T for keys 0-15 (s0) and 16-31 (s1) of the tile
    f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      const bf16x8_t k0f = as_bf16x8(*(const u32x4_t*)&sK[col * LDK + s * 32 + grp * 8]);
      const bf16x8_t k1f = as_bf16x8(*(const u32x4_t*)&sK[(16 + col) * LDK + s * 32 + grp * 8]);
      s0 = mfma16x16x32(k0f, as_bf16x8(qf[s]), s0);
      s1 = mfma16x16x32(k1f, as_bf16x8(qf[s]), s1);
    }
    float mt = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ka = kt + grp * 4 + i, kb2 = ka + 16;
      s0[i] = ka < a.Nk ? s0[i] * sl2 : -INFINITY;
      s1[i] = kb2 < a.Nk ? s1[i] * sl2 : -INFINITY;
      mt = fmaxf(mt, fmaxf(s0[i], s1[i]));
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float mnew = fmaxf(mrun, mt);
    const float alpha = fast_exp2(mrun - mnew);
    float ls = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s0[i] = fast_exp2(s0[i] - mnew);
      s1[i] = fast_exp2(s1[i] - mnew);
      ls += s0[i] + s1[i];
    }
    ls += __shfl_xor(ls, 16, 64);
    ls += __shfl_xor(ls, 32, 64);
    lrun = lrun * alpha + ls;
    mrun = mnew;
    // P^T as the B operand: abstract k = grp * 8 + kk is key (kk / 4) * 16 + grp * 4 + kk % 4
    const u32x4_t pw = {pack_bf2(s0[0], s0[1]), pack_bf2(s0[2], s0[3]), pack_bf2(s1[0], s1[1]), pack_bf2(s1[2], s1[3])};
    const bf16x8_t pf = as_bf16x8(pw);
#pragma unroll
    for (int t2 = 0; t2 < D / 16; ++t2) {
      const uint16_t* row = &sVt[(t2 * 16 + col) * LDV + grp * 4];
      const u32x2_t lo = *(const u32x2_t*)row;
      const u32x2_t hi = *(const u32x2_t*)(row + 16);
      const u32x4_t vw = {lo[0], lo[1], hi[0], hi[1]};
      f32x4_t acc = o[t2];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] *= alpha;
      o[t2] = mfma16x16x32(as_bf16x8(vw), pf, acc);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // merge the four key ranges: m, l and the unnormalised O of every wave through LDS
  __syncthreads();
  float* mb = (float*)lds;   // [4][16]
  float* lb = mb + 64;       // [4][16]
  float* ob = lb + 64;       // [4][16][LDO]
  if (grp == 0) {
    mb[w * 16 + col] = mrun;
    lb[w * 16 + col] = lrun;
  }
#pragma unroll
  for (int t2 = 0; t2 < D / 16; ++t2)
#pragma unroll
    for (int e = 0; e < 4; ++e) ob[(w * 16 + col) * LDO + t2 * 16 + grp * 4 + e] = o[t2][e];
  __syncthreads();
  // every thread owns one column d of the head and walks the 16 queries
  for (int idx = threadIdx.x; idx < 16 * D; idx += 256) {
    const int q = idx / D, d = idx % D;
    const int gq = qb * 16 + q;
    if (gq >= a.Nq) break;  // q only grows along the loop
    float M = mb[q];
#pragma unroll
    for (int ww = 1; ww < 4; ++ww) M = fmaxf(M, mb[ww * 16 + q]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float e = fast_exp2(mb[ww * 16 + q] - M);
      L += e * lb[ww * 16 + q];
      O += e * ob[(ww * 16 + q) * LDO + d];
    }
    const float val = O * __builtin_amdgcn_rcpf(L);
    if (a.o_frag) {
      ((bf16_t*)a.o)[frag_idx(b * a.Nq + gq, j * D + d, a.Hq * D)] = f2bf(val);
    } else {
      const long oi = b * a.o_bs + (long)gq * a.o_rs + (long)j * D + d;
      if (a.o_f32) ((float*)a.o)[oi] = val; else ((bf16_t*)a.o)[oi] = f2bf(val);
    }
  }
}

template <int D>
static hipError_t launch_attn16(const AttnArgs& a, hipStream_t s) {
  const int nQB = (a.Nq + 15) / 16;
  dim3 grid(nQB * a.Hq, a.B);
  hipLaunchKernelGGL(k_attn16<D>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t attention_bf16(const AttnArgs& a, hipStream_t s) {
  if (a.B <= 0 || a.Nq <= 0 || a.Nk <= 0) return hipSuccess;
  if (a.Hq % a.Hkv) return hipErrorInvalidValue;
  if (a.o_frag && (a.o_f32 || a.B * a.Nq > 64)) return hipErrorInvalidValue;
  switch (a.hd) {
    case 64: return launch_attn16<64>(a, s);
    case 128: return launch_attn16<128>(a, s);
    case 256: return launch_attn16<256>(a, s);
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
