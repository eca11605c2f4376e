// Softmax attention of the paper's §III-B, Eq. 2: the prefix is bidirectional
// (every token sees every other), the expert's self-attention covers all chunk
// tokens, and its cross-attention all cached prefix tokens; the only mask is
// key padding, M = -inf for the keys past an observation's prefix length (the
// per-batch klen arrays of AttnArgs).  Query head j reads key/value head
// floor(j * Hkv / Hq).
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
  // finite start: a wave whose keys are all padding then adds exp2(-inf) = 0
  float mrun = -3.0e38f, lrun = 0.f;
  const float sl2 = 1.4426950408889634f / sqrtf((float)D);
  const int nk = a.klen ? min(uniform_ld(a.klen, b), a.Nk) : a.Nk;  // visible keys of this observation

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
    // next tile in flight during this tile's math (the last tile again at the
    // end: an unconditional fetch keeps the wait before each use to one tile)
    fetch(min(t + 1, t1 - 1) * 32);

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
      s0[i] = ka < nk ? s0[i] * sl2 : -INFINITY;
      s1[i] = kb2 < nk ? s1[i] * sl2 : -INFINITY;
      mt = fmaxf(mt, fmaxf(s0[i], s1[i]));
    }
    mt = group4_max(mt);
    // Lazy rescaling: the reference max moves (and O, l are rescaled) only
    // when some query's max grew by more than 8 (log2 units), so weights stay
    // below 2^8 and the rescale of the output registers is rare.  The result
    // O / l does not depend on the reference, only its rounding does.
    const bool grow = mt > mrun + 8.f;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float mnew = grow ? mt : mrun;
      const float alpha = fast_exp2(mrun - mnew);
#pragma unroll
      for (int t2 = 0; t2 < D / 16; ++t2)
#pragma unroll
        for (int e = 0; e < 4; ++e) o[t2][e] *= alpha;
      lrun *= alpha;
      mrun = mnew;
    }
    float ls = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s0[i] = fast_exp2(s0[i] - mrun);
      s1[i] = fast_exp2(s1[i] - mrun);
      ls += s0[i] + s1[i];
    }
    lrun += group4_sum(ls);
    // P^T as the B operand: abstract k = grp * 8 + kk is key (kk / 4) * 16 + grp * 4 + kk % 4
    const u32x4_t pw = {pack_bf2(s0[0], s0[1]), pack_bf2(s0[2], s0[3]), pack_bf2(s1[0], s1[1]), pack_bf2(s1[2], s1[3])};
    const bf16x8_t pf = as_bf16x8(pw);
#pragma unroll
    for (int t2 = 0; t2 < D / 16; ++t2) {
      const uint16_t* row = &sVt[(t2 * 16 + col) * LDV + grp * 4];
      const u32x2_t lo = *(const u32x2_t*)row;
      const u32x2_t hi = *(const u32x2_t*)(row + 16);
      const u32x4_t vw = {lo[0], lo[1], hi[0], hi[1]};
      o[t2] = mfma16x16x32(as_bf16x8(vw), pf, o[t2]);
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
  if (a.Hq % a.Hkv || a.Nk2) return hipErrorInvalidValue;  // one key source only
  if (a.o_frag && (a.o_f32 || a.B * a.Nq > 64)) return hipErrorInvalidValue;
  switch (a.hd) {
    case 64: return launch_attn16<64>(a, s);
    case 128: return launch_attn16<128>(a, s);
    case 256: return launch_attn16<256>(a, s);
    default: return hipErrorInvalidValue;
  }
}

// One 32-key tile of the chunk-style attention for one wave: the transposed
// scores S^T = K Q^T of its 16 queries (keys kt .. kt + 31, those at or past nk
// masked to -inf), the online-softmax update with a lazily moved reference max
// (mrun, lrun), and O^T += V^T P^T with P^T taken from the score registers.
// k holds the tile's 2 * D / 32 key fragments; vf(i) returns value fragment i of
// D / 16 (from registers or from LDS).
template <int D, class VF>
__device__ __forceinline__ void attn_tile(const u32x4_t (&k)[D / 16], VF vf, const u32x4_t (&qf)[D / 32], int kt,
                                          int nk, int grp, float sl2, float& mrun, float& lrun, f32x4_t (&o)[D / 16]) {
  constexpr int KS = D / 32, VS = D / 16;
  f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    s0 = mfma16x16x32(as_bf16x8(k[s]), as_bf16x8(qf[s]), s0);
    s1 = mfma16x16x32(as_bf16x8(k[KS + s]), as_bf16x8(qf[s]), s1);
  }
  float mt = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ka = kt + grp * 4 + i;
    s0[i] = ka < nk ? s0[i] * sl2 : -INFINITY;
    s1[i] = ka + 16 < nk ? s1[i] * sl2 : -INFINITY;
    mt = fmaxf(mt, fmaxf(s0[i], s1[i]));
  }
  mt = group4_max(mt);
  // the reference max moves (and O, l are rescaled) only when some query's
  // max grew by more than 8 (log2 units); weights stay below 2^8
  const bool grow = mt > mrun + 8.f;
  if (__builtin_amdgcn_ballot_w64(grow)) {
    const float mnew = grow ? mt : mrun;
    const float alpha = fast_exp2(mrun - mnew);
#pragma unroll
    for (int t2 = 0; t2 < VS; ++t2)
#pragma unroll
      for (int e = 0; e < 4; ++e) o[t2][e] *= alpha;
    lrun *= alpha;
    mrun = mnew;
  }
  float ls = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s0[i] = fast_exp2(s0[i] - mrun);
    s1[i] = fast_exp2(s1[i] - mrun);
    ls += s0[i] + s1[i];
  }
  lrun += group4_sum(ls);
  const u32x4_t pw = {pack_bf2(s0[0], s0[1]), pack_bf2(s0[2], s0[3]), pack_bf2(s1[0], s1[1]), pack_bf2(s1[2], s1[3])};
  const bf16x8_t pf = as_bf16x8(pw);
#pragma unroll
  for (int t2 = 0; t2 < VS; ++t2) o[t2] = mfma16x16x32(as_bf16x8(vf(t2)), pf, o[t2]);
}

// Merge of the four waves' softmax states (max, sum, unnormalised O^T) of one
// workgroup's 16 rows through LDS in wave order, normalisation and the bf16
// store (row layout or the fragment layout of the next product).  obuf holds
// 4 x 16 rows of D + 4 floats; ends with every wave done with it.
template <int D>
__device__ __forceinline__ void attn_merge_store(const AttnArgs& a, float (*mbuf)[16], float (*lbuf)[16], float* obuf,
                                                 float mrun, float lrun, const f32x4_t (&o)[D / 16], int bx, int by) {
  constexpr int VS = D / 16, LDO = D + 4;
  const int G = a.Hq / a.Hkv, R = G * a.Nq;
  const int g = by % a.Hkv, b = by / a.Hkv;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  if (grp == 0) {
    mbuf[w][col] = mrun;
    lbuf[w][col] = lrun;
  }
#pragma unroll
  for (int t2 = 0; t2 < VS; ++t2) *(f32x4_t*)&obuf[(w * 16 + col) * LDO + t2 * 16 + grp * 4] = o[t2];
  __syncthreads();
  const int qq = threadIdx.x & 15, d0 = (threadIdx.x >> 4) * (D / 16);
  const int r = bx * 16 + qq;
  if (r >= R) return;
  const int jl = r / a.Nq, q = r - jl * a.Nq, j = g * G + jl;
  float M = mbuf[0][qq];
#pragma unroll
  for (int ww = 1; ww < 4; ++ww) M = fmaxf(M, mbuf[ww][qq]);
  float ew[4], L = 0.f;
#pragma unroll
  for (int ww = 0; ww < 4; ++ww) {
    ew[ww] = fast_exp2(mbuf[ww][qq] - M);
    L += ew[ww] * lbuf[ww][qq];
  }
  const float inv = __builtin_amdgcn_rcpf(L);
  const long row = (long)b * a.Nq + q;
#pragma unroll
  for (int d = d0; d < d0 + D / 16; d += 4) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const f32x4_t x = *(const f32x4_t*)&obuf[(ww * 16 + qq) * LDO + d];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += ew[ww] * x[e];
    }
    const u32x2_t pk = {pack_bf2(acc[0] * inv, acc[1] * inv), pack_bf2(acc[2] * inv, acc[3] * inv)};
    const long oi = a.o_frag ? frag_idx((int)row, j * D + d, a.Hq * D) : b * a.o_bs + (long)q * a.o_rs + (long)j * D + d;
    *(u32x2_t*)((bf16_t*)a.o + oi) = pk;
  }
}

// ------------------------------------------------------------------ chunk queries
// attention_chunk: the same attention for short query sets (the action chunk)
// with K and V stored in the MFMA operand orders of common.h (K in frag_idx,
// V in vfrag_idx order, key rows padded to whole 32-key tiles with zero
// values), so every fragment is one contiguous 1 KB wave load straight into
// registers: no LDS staging, no transposes.  All query heads that share a
// key/value head are stacked into R = (Hq / Hkv) * Nq rows (row r is query
// r % Nq of head r / Nq of the group); a workgroup owns 16 rows and its four
// waves take interleaved 32-key tiles (w, w + 4, ...), each with the next
// tile's fragments in flight.  Scores and outputs are formed transposed as in
// k_attn16, with a lazily moved reference max, and the four waves' partial
// softmax states are merged through LDS in wave order.
template <int D>
__global__ __launch_bounds__(256) void k_attn_chunk(AttnArgs a) {
  constexpr int KS = D / 32;  // K fragments per 16 keys
  constexpr int VS = D / 16;  // V fragments per 32-key tile
  constexpr int LDO = D + 4;  // merge rows (floats): 16-lane groups of 16-byte accesses hit distinct banks
  __shared__ float mbuf[4][16], lbuf[4][16];
  __shared__ __attribute__((aligned(16))) float obuf[4][16][LDO];

  if (prefetch_layer(a.pf)) return;  // extra workgroups: warm the next weights
  // (row block, batch and key/value head) of this workgroup; with a multiple of
  // eight of the latter, the workgroups of one observation and head are numbered
  // onto one XCD (the dispatch deals workgroups to the XCDs round robin), so its
  // keys and values are fetched into one L2 instead of all eight
  int bx = blockIdx.x, by = blockIdx.y;
  if ((gridDim.y & 7) == 0) {
    const int L = blockIdx.x + gridDim.x * blockIdx.y, k = L >> 3;
    by = (L & 7) + 8 * (k / gridDim.x);
    bx = k % gridDim.x;
  }
  const int G = a.Hq / a.Hkv, R = G * a.Nq;
  const int g = by % a.Hkv, b = by / a.Hkv;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int r = min(bx * 16 + col, R - 1);  // clamped rows are computed, never stored
  const int jl = r / a.Nq, q = r - jl * a.Nq, j = g * G + jl;
  const bf16_t* Qp = (const bf16_t*)a.q + b * a.q_bs + j * a.q_hs + (long)q * a.q_rs;
  const u32x4_t* Kf = (const u32x4_t*)((const bf16_t*)a.k + b * a.k_bs + g * a.k_hs) + lane;
  const u32x4_t* Vf = (const u32x4_t*)((const bf16_t*)a.v + b * a.v_bs + g * a.v_hs) + lane;
  // joint attention: the second source's tiles follow the first's
  const u32x4_t* Kf2 = a.Nk2 ? (const u32x4_t*)((const bf16_t*)a.k2 + b * a.k2_bs + g * a.k2_hs) + lane : Kf;
  const u32x4_t* Vf2 = a.Nk2 ? (const u32x4_t*)((const bf16_t*)a.v2 + b * a.v2_bs + g * a.v2_hs) + lane : Vf;
  const int TA = (a.Nk + 31) / 32;
  const int T = TA + (a.Nk2 + 31) / 32;
  const int NI = T > w ? (T - 1 - w) / 4 + 1 : 0;  // tiles of this wave (w, w + 4, ...)

  struct Tile { u32x4_t k[2 * KS], v[VS]; };
  auto fetch = [&](Tile& t, int tl) {
    int tile = min(tl, T - 1);
    const bool second = tile >= TA;
    const u32x4_t* kp = second ? Kf2 : Kf;
    const u32x4_t* vp = second ? Vf2 : Vf;
    tile -= second ? TA : 0;
#pragma unroll
    for (int i = 0; i < 2 * KS; ++i) t.k[i] = kp[((long)tile * 2 * KS + i) * 64];
#pragma unroll
    for (int i = 0; i < VS; ++i) t.v[i] = vp[((long)tile * VS + i) * 64];
  };

  u32x4_t qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) qf[s] = *(const u32x4_t*)(Qp + s * 32 + grp * 8);
  Tile ta, tb;

  f32x4_t o[VS];
#pragma unroll
  for (int t = 0; t < VS; ++t) o[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // finite start: a tile whose keys are all masked then adds exp2(-inf) = 0
  float mrun = -3.0e38f, lrun = 0.f;
  const float sl2 = 1.4426950408889634f / sqrtf((float)D);
  // visible keys of this observation in each source (key padding)
  const int nk1 = a.klen ? min(uniform_ld(a.klen, b), a.Nk) : a.Nk;
  const int nk2 = a.klen2 ? min(uniform_ld(a.klen2, b), a.Nk2) : a.Nk2;

  auto consume = [&](const Tile& t, int tl) {
    const bool second = tl >= TA;
    attn_tile<D>(t.k, [&](int i) { return t.v[i]; }, qf, (second ? tl - TA : tl) * 32, second ? nk2 : nk1, grp, sl2,
                 mrun, lrun, o);
  };

  // Tile w + 4 i is consumed from ta (even i) or tb (odd i) while the next is
  // in flight.  A wave fetches only tiles it owns: the kernel's time is largely
  // the bytes one CU pulls through its L1, and with up to three tiles per wave
  // (up to 384 keys) each count has its own straight-line schedule, since
  // branches around the fetches inside one loop cost the compiler registers.
  switch (NI) {
    case 0: break;
    case 1:
      fetch(ta, w);
      consume(ta, w);
      break;
    case 2:
      fetch(ta, w);
      fetch(tb, w + 4);
      consume(ta, w);
      consume(tb, w + 4);
      break;
    case 3:
      fetch(ta, w);
      fetch(tb, w + 4);
      consume(ta, w);
      fetch(ta, w + 8);
      consume(tb, w + 4);
      consume(ta, w + 8);
      break;
    default:  // longer key sets: the last fetches of each buffer are clamped repeats
      fetch(ta, w);
      fetch(tb, w + 4);
      for (int i = 0; i < NI; i += 2) {
        consume(ta, w + 4 * i);
        fetch(ta, w + 4 * (i + 2));
        if (i + 1 >= NI) break;
        consume(tb, w + 4 * (i + 1));
        fetch(tb, w + 4 * (i + 3));
      }
  }

  attn_merge_store<D>(a, mbuf, lbuf, &obuf[0][0][0], mrun, lrun, o, bx, by);
}

// Long key sets with many query rows (batched and multi-camera prefixes): a
// workgroup of four waves owns 64 stacked rows, wave w the 16 rows of row block
// w, and all four walk every 32-key tile, which the workgroup stages once in LDS
// (double-buffered, each wave copying a quarter of it): a CU then pulls the keys
// and values once per 64 rows instead of once per 16.  Each wave keeps its rows'
// softmax state over all keys, so there is no merge: it normalises and stores
// its own rows.  Same tile step, hence the same arithmetic per tile, as
// k_attn_chunk.
template <int D>
__global__ __launch_bounds__(256) void k_attn_rows(AttnArgs a) {
  constexpr int KS = D / 32, VS = D / 16, TF = 2 * KS + VS;  // fragments of one tile: keys, then values
  constexpr int PW = TF / 4;                                 // fragments each wave stages
  __shared__ __attribute__((aligned(16))) u32x4_t kv[2][TF][64];
  int bx = blockIdx.x, by = blockIdx.y;
  if ((gridDim.y & 7) == 0) {  // one observation and head per XCD, as k_attn_chunk
    const int L = blockIdx.x + gridDim.x * blockIdx.y, k = L >> 3;
    by = (L & 7) + 8 * (k / gridDim.x);
    bx = k % gridDim.x;
  }
  const int G = a.Hq / a.Hkv, R = G * a.Nq;
  const int g = by % a.Hkv, b = by / a.Hkv;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int rb = bx * 4 + w;  // this wave's row block
  const int r = min(rb * 16 + col, R - 1);  // clamped rows are computed, never stored
  const int jl = r / a.Nq, q = r - jl * a.Nq, j = g * G + jl;
  const bf16_t* Qp = (const bf16_t*)a.q + b * a.q_bs + j * a.q_hs + (long)q * a.q_rs;
  const u32x4_t* Kf = (const u32x4_t*)((const bf16_t*)a.k + b * a.k_bs + g * a.k_hs) + lane;
  const u32x4_t* Vf = (const u32x4_t*)((const bf16_t*)a.v + b * a.v_bs + g * a.v_hs) + lane;
  const u32x4_t* Kf2 = a.Nk2 ? (const u32x4_t*)((const bf16_t*)a.k2 + b * a.k2_bs + g * a.k2_hs) + lane : Kf;
  const u32x4_t* Vf2 = a.Nk2 ? (const u32x4_t*)((const bf16_t*)a.v2 + b * a.v2_bs + g * a.v2_hs) + lane : Vf;
  const int TA = (a.Nk + 31) / 32;
  const int T = TA + (a.Nk2 + 31) / 32;
  // wave w stages fragments w PW .. w PW + PW - 1 of a tile
  auto gload = [&](u32x4_t (&regs)[PW], int tl) {
    int tile = tl;
    const bool second = tile >= TA;
    const u32x4_t* kp = second ? Kf2 : Kf;
    const u32x4_t* vp = second ? Vf2 : Vf;
    tile -= second ? TA : 0;
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      const int f = w * PW + i;
      regs[i] = f < 2 * KS ? kp[((long)tile * 2 * KS + f) * 64] : vp[((long)tile * VS + f - 2 * KS) * 64];
    }
  };
  auto sstore = [&](const u32x4_t (&regs)[PW], int buf) {
#pragma unroll
    for (int i = 0; i < PW; ++i) kv[buf][w * PW + i][lane] = regs[i];
  };
  u32x4_t qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) qf[s] = *(const u32x4_t*)(Qp + s * 32 + grp * 8);
  f32x4_t o[VS];
#pragma unroll
  for (int t = 0; t < VS; ++t) o[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float mrun = -3.0e38f, lrun = 0.f;
  const float sl2 = 1.4426950408889634f / sqrtf((float)D);
  const int nk1 = a.klen ? min(uniform_ld(a.klen, b), a.Nk) : a.Nk;
  const int nk2 = a.klen2 ? min(uniform_ld(a.klen2, b), a.Nk2) : a.Nk2;
  u32x4_t st[PW];
  gload(st, 0);
  sstore(st, 0);
  __syncthreads();
  for (int t = 0; t < T; ++t) {
    const int buf = t & 1;
    if (t + 1 < T) gload(st, t + 1);  // in flight while this tile is consumed
    u32x4_t kt[2 * KS];
#pragma unroll
    for (int f = 0; f < 2 * KS; ++f) kt[f] = kv[buf][f][lane];
    const bool second = t >= TA;
    attn_tile<D>(kt, [&](int f) { return kv[buf][2 * KS + f][lane]; }, qf, (second ? t - TA : t) * 32,
                 second ? nk2 : nk1, grp, sl2, mrun, lrun, o);
    if (t + 1 < T) sstore(st, buf ^ 1);  // that buffer was last read for tile t - 1, before the barrier below
    __syncthreads();
  }
  if (rb * 16 + col >= R) return;
  // lane (col, grp) holds dims 16 t2 + 4 grp .. + 3 of its row: 8-byte stores
  const float inv = __builtin_amdgcn_rcpf(lrun);
  const long row = (long)b * a.Nq + q;
#pragma unroll
  for (int t2 = 0; t2 < VS; ++t2) {
    const int d = t2 * 16 + grp * 4;
    const u32x2_t pk = {pack_bf2(o[t2][0] * inv, o[t2][1] * inv), pack_bf2(o[t2][2] * inv, o[t2][3] * inv)};
    const long oi = a.o_frag ? frag_idx((int)row, j * D + d, a.Hq * D) : b * a.o_bs + (long)q * a.o_rs + (long)j * D + d;
    *(u32x2_t*)((bf16_t*)a.o + oi) = pk;
  }
}

hipError_t attention_chunk(const AttnArgs& a, hipStream_t s) {
  if (a.B <= 0 || a.Nq <= 0 || a.Nk <= 0) return hipSuccess;
  if (a.Hq % a.Hkv || a.o_f32) return hipErrorInvalidValue;
  if (a.Nk2 < 0 || (a.Nk2 && (!a.k2 || !a.v2))) return hipErrorInvalidValue;
  if (a.pf.blocks < 0 || a.pf.blocks > 1024 || (a.pf.blocks && !a.pf.sink)) return hipErrorInvalidValue;
  const int R = a.Hq / a.Hkv * a.Nq;
  const int per = (R + 15) / 16 * a.Hkv * a.B;
  dim3 grid((R + 15) / 16, a.Hkv * a.B, prefetch_depth(per, a.pf.blocks));
  // at least four 16-row blocks per CU and eight key tiles: 64-row workgroups sharing key tiles through LDS
  const int T = (a.Nk + 31) / 32 + (a.Nk2 + 31) / 32;
  if (!a.pf.blocks && per >= 4 * 256 && T >= 8) {
    const dim3 g4((R + 63) / 64, a.Hkv * a.B);
    switch (a.hd) {
      case 64: hipLaunchKernelGGL(k_attn_rows<64>, g4, dim3(256), 0, s, a); break;
      case 128: hipLaunchKernelGGL(k_attn_rows<128>, g4, dim3(256), 0, s, a); break;
      case 256: hipLaunchKernelGGL(k_attn_rows<256>, g4, dim3(256), 0, s, a); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  switch (a.hd) {
    case 64: hipLaunchKernelGGL(k_attn_chunk<64>, grid, dim3(256), 0, s, a); break;
    case 128: hipLaunchKernelGGL(k_attn_chunk<128>, grid, dim3(256), 0, s, a); break;
    case 256: hipLaunchKernelGGL(k_attn_chunk<256>, grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
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
  // joint attention: the second source's keys follow the first's
  const float* K2 = a.Nk2 ? (const float*)a.k2 + b * a.k2_bs + g * a.k2_hs : K;
  const float* V2 = a.Nk2 ? (const float*)a.v2 + b * a.v2_bs + g * a.v2_hs : V;
  float m = -INFINITY, l = 0.f;
  const int nk1 = a.klen ? min(uniform_ld(a.klen, b), a.Nk) : a.Nk;
  const int nk2 = a.klen2 ? min(uniform_ld(a.klen2, b), a.Nk2) : a.Nk2;
  for (int t = 0; t < a.Nk + a.Nk2; ++t) {
    const bool second = t >= a.Nk;
    const int tt = second ? t - a.Nk : t;
    if (tt >= (second ? nk2 : nk1)) continue;  // key padding: weight 0
    const float* kr = second ? K2 + (long)tt * a.k2_rs : K + (long)tt * a.k_rs;
    float s = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) s = fmaf(qv[d], kr[d], s);
    const float mn = fmaxf(m, s);
    const float al = expf(m - mn), p = expf(s - mn);
    l = l * al + p;
    const float* vr = second ? V2 + (long)tt * a.v2_rs : V + (long)tt * a.v_rs;
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
  if (a.Nk2 < 0 || (a.Nk2 && (!a.k2 || !a.v2))) return hipErrorInvalidValue;
  dim3 grid((a.Nq + 63) / 64, a.Hq, a.B);
  switch (a.hd) {
    case 32: hipLaunchKernelGGL(k_attn_f32<32>, grid, dim3(64), 0, s, a); break;
    case 64: hipLaunchKernelGGL(k_attn_f32<64>, grid, dim3(64), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace vla
