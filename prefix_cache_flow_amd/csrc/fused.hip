// One solver step of the action expert as one persistent kernel (cross
// attention, bf16, at most 64 chunk rows): the row kernel of the step (head of
// the previous step and embedding of this one, the paper's §III-A, Eq. 1), then
// every expert layer's self-attention, cross-attention into the cached K/V
// (§III-B, Eq. 2) and GeGLU MLP, as a fixed sequence of phases.  Each phase is
// the work of one kernel of the kernel-chain path (same tiles, same summation
// orders, so both paths give the same bits); phases are separated by a grid
// barrier instead of a kernel boundary.
//
// Why: at batch 1 a step streams about 770 MB of weights through about 200
// dependent pieces of work.  As a chain of graph kernel nodes each piece pays a
// launch (about 1.65 us) plus a cold start (kernel arguments, first loads from
// HBM); here the workgroups stay resident, each phase starts from data the
// previous phase left in L2, and extra "shadow" workgroups read every compute
// workgroup's next weight tiles into its XCD's L2 two phases ahead.
//
// Coherence across the eight XCDs (each has its own L2): every activation that
// one workgroup writes and another reads goes through device-scope accesses
// (the sc1 cache policy, the same accesses the memory model uses for
// agent-scope atomics), and a workgroup arrives at a barrier only after its
// stores are acknowledged (s_waitcnt vmcnt(0)).  Weights and the K/V cache,
// written by earlier kernels, are read with ordinary loads.
//
// Barrier: each compute workgroup adds 1 to the counter of its group (linear
// id mod 8, which is also the XCD it runs on); the last arrival of a group
// raises that group's flag to the step's generation; everyone waits for all
// eight flags.  Counters and flags are zeroed once per solver run and only
// grow, so one captured graph replays without any reset inside it.  Every wait
// is bounded: after kSpinLimit polls the workgroup records an error and stops
// waiting for the rest of the launch, so a launch always ends.  All compute
// workgroups must be resident at once: the host launches at most one per CU
// times the occupancy it measured.
#include "common.h"
#include "kernels.h"

namespace vla {
namespace {

// tidx() through an empty volatile asm: a fresh, opaque value at every
// use, so the compiler cannot hoist the lane-dependent address arithmetic of
// every phase out of the layer loop and keep it live (and spilled) throughout.
__device__ __forceinline__ int tidx() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// sum over the 256 threads, every thread gets the result (block_sum of common.h)
__device__ __forceinline__ float wg_sum(float v, float* red) {
  v = wave_sum(v);
  const int t = tidx(), w = t >> 6, l = t & 63;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) s += red[i];
  return s;
}

constexpr int kSC1 = 16;                   // cache policy bits: device-scope coherent access
constexpr unsigned kSpinLimit = 1u << 20;  // polls before a barrier wait gives up
constexpr int kBarStride = 9 * 32;         // dwords per barrier: flags line, then 8 counter lines

struct Buf {
  __amdgpu_buffer_rsrc_t r;
};
__device__ __forceinline__ Buf mkbuf(const void* p, uint32_t bytes) {
  Buf b;
  b.r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)min(bytes, 0x7fffffffu), 0x00020000);
  return b;
}
// coherent (device-scope) loads and stores; out-of-range offsets read 0 and drop writes
__device__ __forceinline__ u32x4_t ldc16(const Buf& b, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(b.r, off, 0, kSC1);
}
__device__ __forceinline__ float ldcf(const Buf& b, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(b.r, off, 0, kSC1));
}
__device__ __forceinline__ f32x4_t ldcf4(const Buf& b, uint32_t off) {
  return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(b.r, off, 0, kSC1));
}
__device__ __forceinline__ void stc16(const Buf& b, uint32_t off, u32x4_t v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, b.r, off, 0, kSC1);
}
__device__ __forceinline__ void stc8(const Buf& b, uint32_t off, u32x2_t v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, b.r, off, 0, kSC1);
}
__device__ __forceinline__ void stcf(const Buf& b, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), b.r, off, 0, kSC1);
}
__device__ __forceinline__ void stch(const Buf& b, uint32_t off, bf16_t v) {
  __builtin_amdgcn_raw_buffer_store_b16(v, b.r, off, 0, kSC1);
}

// ---------------------------------------------------------------- grid barrier
__device__ __forceinline__ void gsync(const FusedStepP& p, int b, unsigned gen, bool& dead) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's stores are acknowledged
  __syncthreads();
  if (tidx() < 64) {
    unsigned* base = p.bar + (size_t)b * kBarStride;
    const int x = blockIdx.x & 7;
    if (tidx() == 0) {
      const unsigned nx = (unsigned)((p.nwg - x + 7) >> 3);
      const unsigned old = __hip_atomic_fetch_add(base + 32 * (1 + x), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (old + 1 == gen * nx) __hip_atomic_store(base + x, gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (!dead) {
      const int lane = tidx();
      unsigned spins = 0;
      for (;;) {
        bool ok = true;
        if (lane < 8 && lane < p.nwg) ok = __hip_atomic_load(base + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= gen;
        if (__builtin_amdgcn_ballot_w64(!ok) == 0) break;
        if (++spins > kSpinLimit) {
          if (lane == 0) __hip_atomic_fetch_or(p.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          dead = true;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
  }
  __syncthreads();
}

// wait (shadow workgroups) until barrier b of generation gen has been passed by this group
__device__ __forceinline__ bool wait_flag(const FusedStepP& p, int b, unsigned gen, int group) {
  const unsigned* f = p.bar + (size_t)b * kBarStride + group;
  for (unsigned spins = 0; spins <= kSpinLimit; ++spins) {
    if (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= gen) return true;
    __builtin_amdgcn_s_sleep(4);
  }
  return false;
}

// ---------------------------------------------------------------- GEMM tiles
// The tile of k_chunk (gemm.hip) for column group bx and K chunk by: the four
// waves split the chunk's k-steps, partial tiles are summed through LDS in
// wave order, wave w finishes row block w.  A (activations, fragment layout) is
// read coherently, W (weights, fragment layout) with ordinary loads.
struct GemmT {
  Buf A;
  const u32x4_t* W;
  int M, N, K, kchunk;
  Buf out;
  int ldo;
  Buf kout, vout;  // QKV keys and values (MFMA operand orders)
  int nq, hkv, hd, npre, npad;
  Buf ws;  // PARTIAL [split][M][N]
};

template <int KIND>
__device__ __forceinline__ void gemm_store(const GemmT& p, int m, int n, float v) {
  if (KIND == EPI_STORE) {
    stch(p.out, (uint32_t)(m * p.ldo + n) * 2, f2bf(v));
  } else if (KIND == EPI_QKV) {
    if (n < p.nq) {
      stch(p.out, (uint32_t)(m * p.ldo + n) * 2, f2bf(v));
      return;
    }
    const int per = p.hkv * p.hd;
    const int kv = (n - p.nq) >= per, r = n - p.nq - kv * per;
    const int h = r / p.hd, d = r - h * p.hd;
    const int b = m / p.npre, t = m - b * p.npre;
    const long blk = (long)b * per * p.npad + (long)h * p.npad * p.hd;
    if (kv) stch(p.vout, (uint32_t)(blk + vfrag_idx(t, d, p.hd)) * 2, f2bf(v));
    else stch(p.kout, (uint32_t)(blk + frag_idx(t, d, p.hd)) * 2, f2bf(v));
  }
}

template <int NB, int MB, int KIND, int SPW>
__device__ __forceinline__ void gemm_tile(const GemmT& p, int bx, int by, float* redf) {
  float (*red)[MB * NB * 4][64] = (float (*)[MB * NB * 4][64])redf;
  const int lane = tidx() & 63, w = tidx() >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int nb0 = bx * NB;
  const int KS = p.K >> 5;
  const int sb = (by * p.kchunk + w * (p.kchunk >> 2)) >> 5;
  const int nsteps = max(0, min(KS - sb, p.kchunk >> 7));
  const u32x4_t* Wv = p.W + lane;
  u32x4_t wv[SPW][NB], av[SPW][MB];
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
    const int ks = min(sb + s, KS - 1);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) wv[s][nb] = Wv[((long)(nb0 + nb) * KS + ks) * 64];
#pragma unroll
    for (int rb = 0; rb < MB; ++rb) av[s][rb] = ldc16(p.A, (uint32_t)(((rb * KS + ks) * 64 + lane) * 16));
  }
  f32x4_t acc[MB][NB];
#pragma unroll
  for (int rb = 0; rb < MB; ++rb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[rb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
    const bool on = s < nsteps;
#pragma unroll
    for (int rb = 0; rb < MB; ++rb) {
      const u32x4_t a4 = on ? av[s][rb] : u32x4_t{0, 0, 0, 0};
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[rb][nb] = mfma16x16x32(as_bf16x8(a4), as_bf16x8(wv[s][nb]), acc[rb][nb]);
    }
  }
  __syncthreads();  // the previous user of the LDS area is done
#pragma unroll
  for (int rb = 0; rb < MB; ++rb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int e = 0; e < 4; ++e) red[w][(rb * NB + nb) * 4 + e][lane] = acc[rb][nb][e];
  __syncthreads();
  const int rb = w;
  if (rb < MB) {
    float v[NB][4];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int idx = (rb * NB + nb) * 4 + e;
        v[nb][e] = red[0][idx][lane] + red[1][idx][lane] + red[2][idx][lane] + red[3][idx][lane];
      }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = rb * 16 + grp * 4 + e;
      if (m >= p.M) continue;
      if (KIND == EPI_GEGLU) {
        const int f = (nb0 >> 1) * 16 + col;
        stch(p.out, (uint32_t)frag_idx(m, f, p.ldo) * 2, f2bf(gelu_erf(v[0][e]) * v[NB - 1][e]));
        continue;
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int n = (nb0 + nb) * 16 + col;
        if (KIND == EPI_PARTIAL) stcf(p.ws, (uint32_t)(((long)by * p.M + m) * p.N + n) * 4, v[nb][e]);
        else gemm_store<KIND>(p, m, n, v[nb][e]);
      }
    }
  }
}

// all tiles of one GEMM phase owned by this workgroup (tile t = by * gx + bx)
template <int NB, int MB, int KIND>
__device__ __forceinline__ void gemm_phase(const GemmT& p, int splits, int spw, float* red, int nwg) {
  const int gx = p.N / (16 * NB), T = gx * splits;
  for (int t = blockIdx.x; t < T; t += nwg) {
    const int bx = t % gx, by = t / gx;
    if (spw <= 2) gemm_tile<NB, MB, KIND, 2>(p, bx, by, red);
    else if (spw <= 4) gemm_tile<NB, MB, KIND, 4>(p, bx, by, red);
    else gemm_tile<NB, MB, KIND, 8>(p, bx, by, red);
  }
}

// ---------------------------------------------------------------- attention tiles
// The tile of k_attn_chunk (attention.hip): 16 stacked (head, query) rows of one
// key/value head, four waves over interleaved 32-key tiles, merged through LDS
// in wave order; output in the fragment layout of the O projection.
struct AttnT {
  Buf q;
  long q_bs, q_hs, q_rs;
  Buf k, v;  // whole K / V buffers
  long k_off, v_off;  // element offset of (batch 0, head 0)
  long k_bs, k_hs;    // element strides (same for V)
  Buf o;
  int Nq, Nk, Hq, Hkv, R, nrb;
  const int* klen;  // key padding: visible keys per observation (null: all Nk)
};

template <int D, int AUX>
__device__ __forceinline__ void attn_tile(const AttnT& a, int rbk, int gy, float* lds) {
  constexpr int KS = D / 32, VS = D / 16, LDO = D + 4;
  float* mbuf = lds;                                              // [4][16]
  float* lbuf = lds + 64;                                         // [4][16]
  float (*obuf)[16][LDO] = (float (*)[16][LDO])(lds + 128);       // [4][16][LDO]
  const int G = a.Hq / a.Hkv, R = a.R;
  const int g = gy % a.Hkv, b = gy / a.Hkv;
  const int lane = tidx() & 63, w = tidx() >> 6;
  const int col = lane & 15, grp = lane >> 4;
  int r = min(rbk * 16 + col, R - 1);
  int jl = r / a.Nq, q = r - jl * a.Nq, j = g * G + jl;
  const long qoff = b * a.q_bs + j * a.q_hs + (long)q * a.q_rs;
  const long kb = a.k_off + b * a.k_bs + g * a.k_hs, vb = a.v_off + b * a.k_bs + g * a.k_hs;
  const int T = (a.Nk + 31) / 32;
  const int NI = T > w ? (T - 1 - w) / 4 + 1 : 0;

  struct Tile { u32x4_t k[2 * KS], v[VS]; };
  auto fetch = [&](Tile& t, int tl) {
    const int tile = min(tl, T - 1);
#pragma unroll
    for (int i = 0; i < 2 * KS; ++i)
      t.k[i] = __builtin_amdgcn_raw_buffer_load_b128(a.k.r, (uint32_t)((kb + (((long)tile * 2 * KS + i) * 64 + lane) * 8) * 2), 0, AUX);
#pragma unroll
    for (int i = 0; i < VS; ++i)
      t.v[i] = __builtin_amdgcn_raw_buffer_load_b128(a.v.r, (uint32_t)((vb + (((long)tile * VS + i) * 64 + lane) * 8) * 2), 0, AUX);
  };
  u32x4_t qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) qf[s] = ldc16(a.q, (uint32_t)((qoff + s * 32 + grp * 8) * 2));
  Tile ta, tb;
  f32x4_t o[VS];
#pragma unroll
  for (int t = 0; t < VS; ++t) o[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float mrun = -3.0e38f, lrun = 0.f;
  const float sl2 = 1.4426950408889634f / sqrtf((float)D);
  const int nkb = a.klen ? min(a.klen[b], a.Nk) : a.Nk;

  // scores of tile tl (keys 0-15 in s0, 16-31 in s1), masked and scaled
  auto scores = [&](const Tile& t, int tl, f32x4_t& s0, f32x4_t& s1) {
    s0 = f32x4_t{0.f, 0.f, 0.f, 0.f};
    s1 = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      s0 = mfma16x16x32(as_bf16x8(t.k[s]), as_bf16x8(qf[s]), s0);
      s1 = mfma16x16x32(as_bf16x8(t.k[KS + s]), as_bf16x8(qf[s]), s1);
    }
  };
  // online softmax update and O^T += V^T P^T for one tile's scores
  auto update = [&](const Tile& t, int tl, f32x4_t s0, f32x4_t s1) {
    const int kt = tl * 32, nk = nkb;
    float mt = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ka = kt + grp * 4 + i;
      s0[i] = ka < nk ? s0[i] * sl2 : -INFINITY;
      s1[i] = ka + 16 < nk ? s1[i] * sl2 : -INFINITY;
      mt = fmaxf(mt, fmaxf(s0[i], s1[i]));
    }
    mt = group4_max(mt);
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
    for (int t2 = 0; t2 < VS; ++t2) o[t2] = mfma16x16x32(as_bf16x8(t.v[t2]), pf, o[t2]);
  };
  auto consume = [&](const Tile& t, int tl) {
    f32x4_t s0, s1;
    scores(t, tl, s0, s1);
    update(t, tl, s0, s1);
  };

  if (D >= 256) {
    // one tile in registers: the next tile's keys load once this tile's scores
    // are formed, its values once this tile's P V product is issued
    if (NI > 0) fetch(ta, w);
    for (int i = 0; i < NI; ++i) {
      const int tl = w + 4 * i, tn = min(tl + 4, w + 4 * (NI - 1));
      f32x4_t s0, s1;
      scores(ta, tl, s0, s1);
      if (i + 1 < NI) {
        const int tile = min(tn, T - 1);
#pragma unroll
        for (int j = 0; j < 2 * KS; ++j)
          ta.k[j] = __builtin_amdgcn_raw_buffer_load_b128(a.k.r, (uint32_t)((kb + (((long)tile * 2 * KS + j) * 64 + lane) * 8) * 2), 0, AUX);
      }
      update(ta, tl, s0, s1);
      if (i + 1 < NI) {
        const int tile = min(tn, T - 1);
#pragma unroll
        for (int j = 0; j < VS; ++j)
          ta.v[j] = __builtin_amdgcn_raw_buffer_load_b128(a.v.r, (uint32_t)((vb + (((long)tile * VS + j) * 64 + lane) * 8) * 2), 0, AUX);
      }
    }
  } else {
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
      default:
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
  }
  __syncthreads();  // the previous user of the LDS area is done
  if (grp == 0) {
    mbuf[w * 16 + col] = mrun;
    lbuf[w * 16 + col] = lrun;
  }
#pragma unroll
  for (int t2 = 0; t2 < VS; ++t2) *(f32x4_t*)&obuf[w][col][t2 * 16 + grp * 4] = o[t2];
  __syncthreads();
  const int qq = tidx() & 15, d0 = (tidx() >> 4) * (D / 16);
  r = rbk * 16 + qq;
  if (r < R) {
    jl = r / a.Nq;
    q = r - jl * a.Nq;
    j = g * G + jl;
    float M = mbuf[qq];
#pragma unroll
    for (int ww = 1; ww < 4; ++ww) M = fmaxf(M, mbuf[ww * 16 + qq]);
    float ew[4], L = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      ew[ww] = fast_exp2(mbuf[ww * 16 + qq] - M);
      L += ew[ww] * lbuf[ww * 16 + qq];
    }
    const float inv = __builtin_amdgcn_rcpf(L);
    const int row = b * a.Nq + q;
#pragma unroll
    for (int d = d0; d < d0 + D / 16; d += 4) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) {
        const f32x4_t x = *(const f32x4_t*)&obuf[ww][qq][d];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += ew[ww] * x[e];
      }
      const u32x2_t pk = {pack_bf2(acc[0] * inv, acc[1] * inv), pack_bf2(acc[2] * inv, acc[3] * inv)};
      stc8(a.o, (uint32_t)frag_idx(row, j * D + d, a.Hq * D) * 2, pk);
    }
  }
}

// ---------------------------------------------------------------- residual + RMSNorm rows
// The row of k_resid_norm (norm.hip): h += sum of the split partials in order,
// u = h / sqrt(mean(h^2) + eps) * (1 + gain) to the fragment layout.
template <bool VEC>
__device__ __forceinline__ int row_col(int i) {
  return VEC ? (((int)tidx() + (i >> 2) * 256) << 2) + (i & 3) : (int)tidx() + i * 256;
}

template <int PER, int NS, bool VEC>
__device__ __forceinline__ void norm_row(Buf h, Buf part, int nsplit, int M, int N, const float* gain, float eps, Buf u, bool write_u,
                         int m, float* red) {
  constexpr int G = VEC ? 4 : 1;
  float x[PER];
  float pv[NS > 0 ? NS : 1][PER];
  float ss = 0.f;
  auto load = [&](const Buf& bb, long rowoff, float* dst) {
#pragma unroll
    for (int i = 0; i < PER; i += G) {
      if (VEC) {
        const f32x4_t v = ldcf4(bb, (uint32_t)((rowoff + row_col<true>(i)) * 4));
#pragma unroll
        for (int j = 0; j < 4; ++j) dst[i + j] = v[j];
      } else {
        dst[i] = ldcf(bb, (uint32_t)((rowoff + min(row_col<false>(i), N - 1)) * 4));
      }
    }
  };
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
  load(h, (long)m * N, x);
#pragma unroll
  for (int s = 0; s < NS; ++s) load(part, ((long)min(s, nsplit - 1) * M + m) * N, pv[s]);
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
      if (VEC) {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, f32x4_t{x[i], x[i + 1], x[i + 2], x[i + 3]}),
                                               h.r, (uint32_t)(((long)m * N + n) * 4), 0, kSC1);
      } else if (n < N) {
        stcf(h, (uint32_t)(((long)m * N + n) * 4), x[i]);
      }
    }
  }
  ss = wg_sum(ss, red);
  const float r = 1.0f / sqrtf(ss / (float)N + eps);
#pragma unroll
  for (int i = 0; i < PER; ++i) x[i] = x[i] * r * gk[i];
  if (write_u) {
#pragma unroll
    for (int i = 0; i < PER; i += G) {
      const int n = row_col<VEC>(i);
      if (VEC) {
        stc8(u, (uint32_t)frag_idx(m, n, N) * 2, u32x2_t{pack_bf2(x[i], x[i + 1]), pack_bf2(x[i + 2], x[i + 3])});
      } else if (n < N) {
        stch(u, (uint32_t)frag_idx(m, n, N) * 2, f2bf(x[i]));
      }
    }
  }
}

// nsplit <= 4 and N <= 1024 (the host only takes this path then)
template <int PER, bool VEC>
__device__ __forceinline__ void norm_rows_ns(Buf h, Buf part, int nsplit, int M, int N, const float* gain, float eps,
                                             Buf u, bool write_u, float* red, int nwg) {
  for (int m = blockIdx.x; m < M; m += nwg) {
    if (nsplit <= 1) norm_row<PER, 1, VEC>(h, part, nsplit, M, N, gain, eps, u, write_u, m, red);
    else norm_row<PER, 4, VEC>(h, part, nsplit, M, N, gain, eps, u, write_u, m, red);
  }
}

__device__ __forceinline__ void norm_phase(Buf h, Buf part, int nsplit, int M, int N, const float* gain, float eps,
                                           Buf u, bool write_u, float* red, int nwg) {
  const int per = (N + 255) / 256;
  if (per <= 1) norm_rows_ns<1, false>(h, part, nsplit, M, N, gain, eps, u, write_u, red, nwg);
  else if (per <= 2) norm_rows_ns<2, false>(h, part, nsplit, M, N, gain, eps, u, write_u, red, nwg);
  else if (N % 1024 == 0) norm_rows_ns<4, true>(h, part, nsplit, M, N, gain, eps, u, write_u, red, nwg);
  else norm_rows_ns<4, false>(h, part, nsplit, M, N, gain, eps, u, write_u, red, nwg);
}

// ---------------------------------------------------------------- step rows
// The row of k_step_rows (expert.hip): velocity head of step k_head with the
// Euler update, then the embedding of step k_embed with the first layer's
// RMSNorm.  FH / FE select the fast forms (bf16 weights, d_e <= 1024,
// d_a <= 32; the head also d_e % 64 == 0, the embedding d_a % 8 == 0), exactly
// as the row kernel picks them.
template <bool FH, bool FE>
__device__ __forceinline__ void step_row(const FusedStepP& a, int m, int k_head, int k_embed, float* us, float* xs, float* red) {
  const int tid = tidx();
  const bool head = k_head >= 0, emb = k_embed >= 0;
  const Buf Eb = mkbuf(a.E, a.bytes_E), Xb = mkbuf(a.X, a.bytes_X), Ub = mkbuf(a.u, a.bytes_u);
  constexpr int G = 8;
  const int part = tid % G, ao = tid / G;
  constexpr int PER = 4;
  u32x4_t wo[16], wi[16];
  float er[PER], gf[PER], g1[PER];
  const float dt = head ? a.sched[k_head + 1] - a.sched[k_head] : 0.f;
  const float tau = emb ? a.sched[k_embed] : 0.f;
  const bool xown = FH && head && part == 0 && ao < a.d_a;
  const float x0 = xown ? ldcf(Xb, (uint32_t)((m * a.d_a + ao) * 4)) : 0.f;
  if (FH && head) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int n = min(tid + i * 256, a.d_e - 1);
      er[i] = ldcf(Eb, (uint32_t)((m * a.d_e + n) * 4));
      gf[i] = a.w_ef[n];
    }
  }
  if (FE && emb) {
#pragma unroll
    for (int i = 0; i < PER; ++i) g1[i] = a.egains[min(tid + i * 256, a.d_e - 1)];
  }
  if (FH && head) {
    const int sl = a.d_e / G;
    const bf16_t* wr = a.w_out + (long)min(ao, a.d_a - 1) * a.d_e + part * sl;
#pragma unroll
    for (int t = 0; t < 16; ++t) wo[t] = *(const u32x4_t*)(wr + min(t * 8, sl - 8));
  }
  if (FE && emb) {
    const int dv = a.d_a / 8;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int i = t / 4, v = t % 4;
      const int n = min(tid + i * 256, a.d_e - 1);
      wi[t] = *(const u32x4_t*)(a.w_in + (long)n * a.d_a + min(v, dv - 1) * 8);
    }
  }
  __syncthreads();  // the previous user of the LDS area is done
  if (head) {
    float ss = 0.f;
    if (FH) {
#pragma unroll
      for (int i = 0; i < PER; ++i) ss = fmaf(er[i], tid + i * 256 < a.d_e ? er[i] : 0.f, ss);
      ss = wg_sum(ss, red);
      const float r = 1.0f / sqrtf(ss / (float)a.d_e + a.eps);
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if (tid + i * 256 < a.d_e) us[tid + i * 256] = er[i] * r * (1.0f + gf[i]);
    } else {
      for (int n = tid; n < a.d_e; n += 256) {
        const float v = ldcf(Eb, (uint32_t)((m * a.d_e + n) * 4));
        us[n] = v;
        ss = fmaf(v, v, ss);
      }
      ss = wg_sum(ss, red);
      const float r = 1.0f / sqrtf(ss / (float)a.d_e + a.eps);
      for (int n = tid; n < a.d_e; n += 256) us[n] = us[n] * r * (1.0f + a.w_ef[n]);
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
        for (int hh = 0; hh < 4; ++hh) {
          acc = fmaf(ur[2 * hh], bf2f((bf16_t)(wo[t][hh] & 0xffffu)), acc);
          acc = fmaf(ur[2 * hh + 1], bf2f((bf16_t)(wo[t][hh] >> 16)), acc);
        }
      }
#pragma unroll
      for (int o = 1; o < G; o <<= 1) acc += __shfl_xor(acc, o, 64);
      if (xown) {
        const float x = x0 + dt * acc;
        stcf(Xb, (uint32_t)((m * a.d_a + ao) * 4), x);
        xs[ao] = x;
      }
    } else {
      for (int o = ao; o < a.d_a; o += 256 / G) {
        float acc = 0.f;
        for (int n = part; n < a.d_e; n += G) acc = fmaf(us[n], bf2f(a.w_out[(long)o * a.d_e + n]), acc);
#pragma unroll
        for (int qq = 1; qq < G; qq <<= 1) acc += __shfl_xor(acc, qq, 64);
        if (part == 0) {
          const float x = ldcf(Xb, (uint32_t)((m * a.d_a + o) * 4)) + dt * acc;
          stcf(Xb, (uint32_t)((m * a.d_a + o) * 4), x);
          xs[o] = x;
        }
      }
    }
  } else if (tid < a.d_a) {
    xs[tid] = ldcf(Xb, (uint32_t)((m * a.d_a + tid) * 4));
  }
  if (!emb) return;
  __syncthreads();
  const float l2 = 13.287712379549449f;  // log2(10000)
  float ss = 0.f;
  auto emit = [&](int n, float v) {
    const float freq = fast_exp2(-l2 * (2.0f * (float)(n >> 1) / (float)a.d_e));
    const float arg = tau * freq;
    v += (n & 1) ? __cosf(arg) : __sinf(arg);
    stcf(Eb, (uint32_t)((m * a.d_e + n) * 4), v);
    us[n] = v;
    ss = fmaf(v, v, ss);
  };
  if (FE) {
    const int dv = a.d_a / 8;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int n = tid + i * 256;
      if (n >= a.d_e) break;
      float v = 0.f;
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        if (qd >= dv) break;
        const u32x4_t w = wi[i * 4 + qd];
#pragma unroll
        for (int hh = 0; hh < 4; ++hh) {
          v = fmaf(xs[qd * 8 + 2 * hh], bf2f((bf16_t)(w[hh] & 0xffffu)), v);
          v = fmaf(xs[qd * 8 + 2 * hh + 1], bf2f((bf16_t)(w[hh] >> 16)), v);
        }
      }
      emit(n, v);
    }
  } else {
    for (int n = tid; n < a.d_e; n += 256) {
      float v = 0.f;
      for (int a0 = 0; a0 < a.d_a; ++a0) v = fmaf(xs[a0], bf2f(a.w_in[(long)n * a.d_a + a0]), v);
      emit(n, v);
    }
  }
  ss = wg_sum(ss, red);
  const float r = 1.0f / sqrtf(ss / (float)a.d_e + a.eps);
  auto put_u = [&](int n, float g) { stch(Ub, (uint32_t)frag_idx(m, n, a.d_e) * 2, f2bf(us[n] * r * (1.0f + g))); };
  if (FE) {
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (tid + i * 256 < a.d_e) put_u(tid + i * 256, g1[i]);
  } else {
    for (int n = tid; n < a.d_e; n += 256) put_u(n, a.egains[n]);
  }
}

__device__ __forceinline__ void rows_phase(const FusedStepP& a, int k_head, int k_embed, float* us, float* xs, float* red) {
  if (k_head < 0 && k_embed < 0) return;
  const bool fh = a.d_e % 64 == 0 && a.d_e <= 1024 && a.d_a <= 32;
  const bool fe = a.d_a % 8 == 0 && a.d_a <= 32 && a.d_e <= 1024;
  for (int m = blockIdx.x; m < a.M; m += a.nwg) {
    if (fh && fe) step_row<true, true>(a, m, k_head, k_embed, us, xs, red);
    else if (fh) step_row<true, false>(a, m, k_head, k_embed, us, xs, red);
    else if (fe) step_row<false, true>(a, m, k_head, k_embed, us, xs, red);
    else step_row<false, false>(a, m, k_head, k_embed, us, xs, red);
  }
}

// ---------------------------------------------------------------- shadow workgroups
// Read the fragment-layout weight ranges of the tiles that compute workgroup
// `cw` owns in a GEMM phase, so they are in its XCD's L2 when it gets there.
__device__ __forceinline__ void warm_gemm(const u32x4_t* W, int N, int K, int kchunk, int splits, int NB, int cw, int nwg) {
  const int gx = N / (16 * NB), T = gx * splits, KS = K >> 5;
  unsigned x = 0;
  for (int t = cw; t < T; t += nwg) {
    const int bx = t % gx, by = t / gx;
    const int k0 = (by * kchunk) >> 5, k1 = min(KS, ((by + 1) * kchunk) >> 5);
    if (k1 <= k0) continue;
    const int nvec = (k1 - k0) * 64;  // 16-byte vectors per column block
    for (int nb = 0; nb < NB; ++nb) {
      const u32x4_t* base = W + ((long)(bx * NB + nb) * KS + k0) * 64;
      for (int i0 = tidx(); i0 < nvec; i0 += 256 * 8) {
        u32x4_t t8[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) t8[u] = base[min(i0 + u * 256, nvec - 1)];
#pragma unroll
        for (int u = 0; u < 8; ++u) x ^= t8[u][0] ^ t8[u][3];
      }
    }
  }
  if (x == 0x9E3779B9u) __builtin_amdgcn_s_sleep(1);  // keeps the loads
}

__device__ __forceinline__ void warm_range(const void* p, long bytes) {
  const u32x4_t* v = (const u32x4_t*)p;
  const long n = bytes >> 4;
  unsigned x = 0;
  for (long i0 = tidx(); i0 < n; i0 += 256 * 8) {
    u32x4_t t8[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) t8[u] = v[min(i0 + u * 256, n - 1)];
#pragma unroll
    for (int u = 0; u < 8; ++u) x ^= t8[u][0] ^ t8[u][3];
  }
  if (x == 0x9E3779B9u) __builtin_amdgcn_s_sleep(1);
}

}  // namespace

// ---------------------------------------------------------------- the kernel
// Phase order of one layer: self QKV, self attention, self O (split partials),
// residual + norm, cross Q, cross attention, cross O (partials), residual +
// norm, gate/up + GeGLU, down (partials), residual + norm.  Barrier b of a
// step: 0 after the row phase, then 1 + 11 l + i after phase i of layer l.
template <int D, int MB>
__global__ __launch_bounds__(256, 2) void k_fused_step(FusedStepP p) {
  constexpr int kRed = 4 * MB * 2 * 4 * 64;          // GEMM partial tiles (floats)
  constexpr int kAttn = 128 + 4 * 16 * (D + 4);      // attention merge (floats)
  constexpr int kRows = 4096 + 256 + 8;              // step rows
  constexpr int kLds = kRed > kAttn ? (kRed > kRows ? kRed : kRows) : (kAttn > kRows ? kAttn : kRows);
  __shared__ __attribute__((aligned(16))) float lds[kLds];
  const int nwg = p.nwg;
  const int L = p.L, qe = p.qe, qkve = p.qkve, d_e = p.d_e, F = p.F;
  const long ewl = p.ew_layer;

  if ((int)blockIdx.x >= nwg) {
    // shadow workgroup of compute workgroup cw (same group, so same XCD, as
    // cw): reads cw's weight tiles of a phase while the phases before it run
    const int cw = blockIdx.x - nwg, grp = cw & 7;
    for (int l = 0; l < L; ++l) {
      const char* lw = p.ew + l * ewl;
      const int b0 = 1 + 11 * l;
      if (l > 0 && !wait_flag(p, b0 - 3, p.gen, grp)) return;  // previous gate/up done
      warm_gemm((const u32x4_t*)(lw + p.off_qkv), qkve, d_e, p.kc_qkv, 1, 1, cw, nwg);
      if (!wait_flag(p, b0, p.gen, grp)) return;  // QKV done
      warm_gemm((const u32x4_t*)(lw + p.off_os), d_e, qe, p.kc_o, p.s_o, 1, cw, nwg);
      if (!wait_flag(p, b0 + 2, p.gen, grp)) return;  // self O done
      warm_gemm((const u32x4_t*)(lw + p.off_qc), qe, d_e, p.kc_q, 1, 1, cw, nwg);
      if (cw < p.nrb * p.Hkv * p.B && p.B == 1)
        warm_range(p.cache + (long)l * 2 * p.Hkv * p.Np * D, (long)2 * p.Hkv * p.Np * D * 2);
      if (!wait_flag(p, b0 + 4, p.gen, grp)) return;  // cross Q done
      warm_gemm((const u32x4_t*)(lw + p.off_oc), d_e, qe, p.kc_o, p.s_o, 1, cw, nwg);
      if (!wait_flag(p, b0 + 6, p.gen, grp)) return;  // cross O done
      warm_gemm((const u32x4_t*)(lw + p.off_gu), 2 * F, d_e, p.kc_gu, 1, 2, cw, nwg);
      if (!wait_flag(p, b0 + 7, p.gen, grp)) return;  // norm before the MLP done
      warm_gemm((const u32x4_t*)(lw + p.off_d), d_e, F, p.kc_d, p.s_d, 1, cw, nwg);
    }
    return;
  }

  bool dead = false;
  const unsigned gen = p.gen;
  const Buf Eb = mkbuf(p.E, p.bytes_E), Ub = mkbuf(p.u, p.bytes_u), Qb = mkbuf(p.q, p.bytes_q);
  const Buf Kb = mkbuf(p.kc, p.bytes_kv), Vb = mkbuf(p.vc, p.bytes_kv), Ab = mkbuf(p.attn, p.bytes_attn);
  const Buf Cq = mkbuf(p.eq, p.bytes_q), Gb = mkbuf(p.g, p.bytes_g), Pb = mkbuf(p.part, p.bytes_part);
  const Buf Cb = mkbuf(p.cache, p.bytes_cache);

  rows_phase(p, p.k_head, p.k_embed, lds, lds + 4096, lds + 4096 + 256);
  gsync(p, 0, gen, dead);

  GemmT gq{};  // self QKV
  gq.A = Ub; gq.M = p.M; gq.N = qkve; gq.K = d_e; gq.kchunk = p.kc_qkv;
  gq.out = Qb; gq.ldo = qe; gq.kout = Kb; gq.vout = Vb; gq.nq = qe; gq.hkv = p.Hkv; gq.hd = D; gq.npre = p.H;
  gq.npad = p.Hp;
  GemmT go{};  // self / cross O: partials
  go.A = Ab; go.M = p.M; go.N = d_e; go.K = qe; go.kchunk = p.kc_o; go.ws = Pb;
  GemmT gc{};  // cross Q
  gc.A = Ub; gc.M = p.M; gc.N = qe; gc.K = d_e; gc.kchunk = p.kc_q; gc.out = Cq; gc.ldo = qe;
  GemmT gg{};  // gate/up + GeGLU
  gg.A = Ub; gg.M = p.M; gg.N = 2 * F; gg.K = d_e; gg.kchunk = p.kc_gu; gg.out = Gb; gg.ldo = F;
  GemmT gd{};  // down: partials
  gd.A = Gb; gd.M = p.M; gd.N = d_e; gd.K = F; gd.kchunk = p.kc_d; gd.ws = Pb;

  AttnT sa{};
  sa.q = Qb; sa.q_bs = (long)p.H * qe; sa.q_hs = D; sa.q_rs = qe;
  sa.k = Kb; sa.v = Vb; sa.k_off = 0; sa.v_off = 0; sa.k_bs = (long)p.Hkv * p.Hp * D; sa.k_hs = (long)p.Hp * D;
  sa.o = Ab; sa.Nq = p.H; sa.Nk = p.H; sa.Hq = p.Hq; sa.Hkv = p.Hkv; sa.R = p.Hq / p.Hkv * p.H; sa.nrb = p.nrb;
  AttnT ca = sa;
  ca.q = Cq; ca.k = Cb; ca.v = Cb; ca.k_bs = (long)L * 2 * p.Hkv * p.Np * D; ca.k_hs = (long)p.Np * D; ca.Nk = p.N;
  ca.klen = p.klen;
  const int nat = p.nrb * p.Hkv * p.B;  // attention tiles

  for (int l = 0; l < L; ++l) {
    const char* lw = p.ew + l * ewl;
    const float* gains = p.egains + (long)l * 3 * d_e;
    const int b0 = 1 + 11 * l;
    gq.W = (const u32x4_t*)(lw + p.off_qkv);
    gemm_phase<1, MB, EPI_QKV>(gq, 1, p.spw_qkv, lds, nwg);
    gsync(p, b0, gen, dead);
    for (int t = blockIdx.x; t < nat; t += nwg) attn_tile<D, kSC1>(sa, t % p.nrb, t / p.nrb, lds);
    gsync(p, b0 + 1, gen, dead);
    go.W = (const u32x4_t*)(lw + p.off_os);
    gemm_phase<1, MB, EPI_PARTIAL>(go, p.s_o, p.spw_o, lds, nwg);
    gsync(p, b0 + 2, gen, dead);
    norm_phase(Eb, Pb, p.s_o, p.M, d_e, gains + d_e, p.eps, Ub, true, lds, nwg);
    gsync(p, b0 + 3, gen, dead);
    gc.W = (const u32x4_t*)(lw + p.off_qc);
    gemm_phase<1, MB, EPI_STORE>(gc, 1, p.spw_q, lds, nwg);
    gsync(p, b0 + 4, gen, dead);
    ca.k_off = (long)l * 2 * p.Hkv * p.Np * D;
    ca.v_off = ca.k_off + (long)p.Hkv * p.Np * D;
    for (int t = blockIdx.x; t < nat; t += nwg) attn_tile<D, 0>(ca, t % p.nrb, t / p.nrb, lds);
    gsync(p, b0 + 5, gen, dead);
    go.W = (const u32x4_t*)(lw + p.off_oc);
    gemm_phase<1, MB, EPI_PARTIAL>(go, p.s_o, p.spw_o, lds, nwg);
    gsync(p, b0 + 6, gen, dead);
    norm_phase(Eb, Pb, p.s_o, p.M, d_e, gains + 2 * d_e, p.eps, Ub, true, lds, nwg);
    gsync(p, b0 + 7, gen, dead);
    gg.W = (const u32x4_t*)(lw + p.off_gu);
    gemm_phase<2, MB, EPI_GEGLU>(gg, 1, p.spw_gu, lds, nwg);
    gsync(p, b0 + 8, gen, dead);
    gd.W = (const u32x4_t*)(lw + p.off_d);
    gemm_phase<1, MB, EPI_PARTIAL>(gd, p.s_d, p.spw_d, lds, nwg);
    gsync(p, b0 + 9, gen, dead);
    const bool last = l + 1 == L;
    norm_phase(Eb, Pb, p.s_d, p.M, d_e, last ? p.w_ef : p.egains + (long)(l + 1) * 3 * d_e, p.eps, Ub, !last, lds, nwg);
    if (!last || p.trailing_head) gsync(p, b0 + 10, last ? p.gen_tail : gen, dead);
  }
  if (p.trailing_head) rows_phase(p, p.k_tail, -1, lds, lds + 4096, lds + 4096 + 256);
}

// ---------------------------------------------------------------- host side
__global__ void k_zero_words(unsigned* p, long n) {
  for (long i = blockIdx.x * (long)blockDim.x + tidx(); i < n; i += (long)gridDim.x * blockDim.x) p[i] = 0u;
}

long fused_barrier_words(int L) { return (long)(2 + 11 * L) * kBarStride; }

hipError_t fused_zero(unsigned* bar, long words, hipStream_t s) {
  if (words <= 0) return hipSuccess;
  const int blocks = (int)std::min<long>((words + 255) / 256, 1024);
  hipLaunchKernelGGL(k_zero_words, dim3(blocks), dim3(256), 0, s, bar, words);
  return hipGetLastError();
}

template <int D, int MB>
static const void* fused_fn() {
  return (const void*)k_fused_step<D, MB>;
}

static const void* fused_kernel(int D, int MB) {
  switch (D) {
    case 64: return MB == 1 ? fused_fn<64, 1>() : MB == 2 ? fused_fn<64, 2>() : fused_fn<64, 4>();
    case 128: return MB == 1 ? fused_fn<128, 1>() : MB == 2 ? fused_fn<128, 2>() : fused_fn<128, 4>();
    case 256: return MB == 1 ? fused_fn<256, 1>() : MB == 2 ? fused_fn<256, 2>() : fused_fn<256, 4>();
  }
  return nullptr;
}

int fused_occupancy(int D, int M) {
  const void* f = fused_kernel(D, M <= 16 ? 1 : M <= 32 ? 2 : 4);
  if (!f) return 0;
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, f, 256, 0) != hipSuccess) return 0;
  return occ;
}

hipError_t fused_step(const FusedStepP& p, int shadows, hipStream_t s) {
  const int MB = p.M <= 16 ? 1 : p.M <= 32 ? 2 : 4;
  const void* f = fused_kernel(p.D, MB);
  if (!f || p.nwg <= 0) return hipErrorInvalidValue;
  FusedStepP a = p;
  void* args[] = {&a};
  return hipLaunchKernel(f, dim3(p.nwg + (shadows ? p.nwg : 0)), dim3(256), args, 0, s);
}

}  // namespace vla
