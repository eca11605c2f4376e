// Dense projections of the policy step: C = A W^T with A [M, K] activations and
// W [N, K] weights (the [out, in] layout of every linear layer).
//
// gemm_frag (the prefix, and any bf16 product of more than 64 rows with both
//   operands in the fragment layout of common.h): 288-row tiles, k_gemm_af8 /
//   k_gemm_af.  Output tiles are numbered XCD-major so tiles that share a
//   weight panel or an activation K range run on one XCD and share its L2.
// gemm_chunk (at most 64 rows, fragment layout): weight-streaming k_chunk.
//   Split-K writes fp32 partials [split][M][N] that a fixed-order reduction (or
//   the row kernel of norm.hip) sums, so results never depend on timing.
// gemm_f32: fp32 SIMT tiles for the fp32 workload (small shapes).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace vla {

__device__ __forceinline__ void cache_index(const Epilogue& e, int m, int n, long& idx) {
  const int per_kv = e.hkv * e.hd, per_l = 2 * per_kv;
  const int l = n / per_l;
  int r = n - l * per_l;
  const int kv = r / per_kv;
  r -= kv * per_kv;
  const int h = r / e.hd, d = r - h * e.hd;
  const int b = m / e.npre, t = m - b * e.npre;
  const long blk = ((((long)(b * e.L + l) * 2 + kv) * e.hkv + h) * e.npad) * e.hd;
  idx = blk + (!e.out_frag ? (long)t * e.hd + d : kv ? vfrag_idx(t, d, e.hd) : frag_idx(t, d, e.hd));
}

// EPI_CACHE with vcopy (bf16, one observation): a value also goes to the copy
// in frag_idx order, the operand order for products that contract over hd
__device__ __forceinline__ void cache_vcopy(const Epilogue& e, int m, int n, float v) {
  const int per_kv = e.hkv * e.hd, per_l = 2 * per_kv;
  const int l = n / per_l;
  int r = n - l * per_l - per_kv;
  if (r < 0) return;  // a key
  const int h = r / e.hd, d = r - h * e.hd;
  ((bf16_t*)e.vcopy)[(long)(l * e.hkv + h) * e.npad * e.hd + frag_idx(m, d, e.hd)] = f2bf(v);
}

// EPI_QKV: query columns to rows, keys and values in their blocks (bf16: MFMA orders)
__device__ __forceinline__ void qkv_store(const Epilogue& e, int m, int n, float v) {
  if (n < e.nq) {
    const long i = (long)m * e.ldo + n;
    if (e.out_f32) ((float*)e.out)[i] = v; else ((bf16_t*)e.out)[i] = f2bf(v);
    return;
  }
  const int per = e.hkv * e.hd;
  const int kv = (n - e.nq) >= per, r = n - e.nq - kv * per;
  const int h = r / e.hd, d = r - h * e.hd;
  const int b = m / e.npre, t = m - b * e.npre;
  const long bs = e.kv_bs ? e.kv_bs : (long)per * e.npad;
  const long blk = b * bs + (long)h * e.npad * e.hd;
  if (e.out_f32) ((float*)(kv ? e.vout : e.kout))[blk + (long)t * e.hd + d] = v;
  else if (kv) ((bf16_t*)e.vout)[blk + vfrag_idx(t, d, e.hd)] = f2bf(v);
  else ((bf16_t*)e.kout)[blk + frag_idx(t, d, e.hd)] = f2bf(v);
}

// Store one finished element (every kind but GEGLU, which needs a pair).  The
// kind is a template parameter so a kernel carries only its own store path:
// kernels here start with a cold instruction cache, and in a chain of short
// kernels their code size is latency.
template <int KIND>
__device__ __forceinline__ void epi_store_t(const Epilogue& e, int m, int n, float v) {
  if (KIND == EPI_STORE) {
    const long i = (long)m * e.ldo + n;
    if (e.out_f32) ((float*)e.out)[i] = v; else ((bf16_t*)e.out)[i] = f2bf(v);
  } else if (KIND == EPI_RESID) {
    e.resid[(long)m * e.ldr + n] += v;
  } else if (KIND == EPI_CACHE) {
    long i;
    cache_index(e, m, n, i);
    if (e.out_f32) ((float*)e.out)[i] = v; else ((bf16_t*)e.out)[i] = f2bf(v);
    if (e.vcopy) cache_vcopy(e, m, n, v);
  } else if (KIND == EPI_QKV) {
    qkv_store(e, m, n, v);
  }
}

__device__ __forceinline__ void epi_store(const Epilogue& e, int m, int n, float v) {
  if (e.kind == EPI_STORE) epi_store_t<EPI_STORE>(e, m, n, v);
  else if (e.kind == EPI_RESID) epi_store_t<EPI_RESID>(e, m, n, v);
  else if (e.kind == EPI_CACHE) epi_store_t<EPI_CACHE>(e, m, n, v);
  else if (e.kind == EPI_QKV) epi_store_t<EPI_QKV>(e, m, n, v);
}

__device__ __forceinline__ void epi_geglu(const Epilogue& e, int m, int f, float g, float u) {
  const float v = gelu_erf(g) * u;
  const long i = e.out_frag ? frag_idx(m, f, e.ldo) : (long)m * e.ldo + f;
  if (e.out_f32) ((float*)e.out)[i] = v; else ((bf16_t*)e.out)[i] = f2bf(v);
}

// Fixed-order sum of split-K partials followed by the epilogue.  Except for
// GeGLU (which pairs columns 16 apart), a thread takes four consecutive
// columns of a row with 16-byte partial loads (N % 4 == 0 for every caller).
__global__ __launch_bounds__(256) void k_splitk_reduce(const float* ws, int splits, int M, int N, Epilogue e) {
  if (e.kind != EPI_GEGLU) {
    const long total4 = (long)M * N / 4, slab = (long)M * N;
    for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < total4; i += (long)gridDim.x * blockDim.x) {
      f32x4_t v = *(const f32x4_t*)(ws + 4 * i);
      for (int s = 1; s < splits; ++s) v += *(const f32x4_t*)(ws + s * slab + 4 * i);
      const int m = (int)(4 * i / N), n = (int)(4 * i % N);
      if (e.kind == EPI_STORE && !e.out_f32) {
        *(u32x2_t*)((bf16_t*)e.out + (long)m * e.ldo + n) = u32x2_t{pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3])};
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) epi_store(e, m, n + j, v[j]);
      }
    }
    return;
  }
  const long total = (long)M * (N / 2);
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < total; i += (long)gridDim.x * blockDim.x) {
    {
      const int F = N / 2;
      const int m = (int)(i / F), f = (int)(i % F);
      const int ng = (f >> 4) * 32 + (f & 15), nu = ng + 16;
      float g = 0.f, u = 0.f;
      for (int s = 0; s < splits; ++s) {
        g += ws[((long)s * M + m) * N + ng];
        u += ws[((long)s * M + m) * N + nu];
      }
      epi_geglu(e, m, f, g, u);
    }
  }
}


// ------------------------------------------------------------------ chunk split planning
constexpr int kChunkSteps = 8;  // at most this many k-steps of 32 per wave

// K is cut into `used` workgroup chunks of a multiple of 4 k-steps each and at
// most 4 * kChunkSteps k-steps; `splits` asks for more chunks than that floor.
static void chunk_plan(int K, int splits, int* used, int* per_steps) {
  const int steps = K / 32;
  const int cap = 4 * kChunkSteps;
  int u0 = std::max((steps + cap - 1) / cap, std::min(std::max(splits, 1), (steps + 3) / 4));
  u0 = std::max(u0, 1);
  int per = (steps + u0 - 1) / u0;
  per = (per + 3) / 4 * 4;
  *per_steps = per;
  *used = (steps + per - 1) / per;
}

void gemm_chunk_plan(int K, int splits, int* used, int* kchunk) {
  int per = 0;
  chunk_plan(K, splits, used, &per);
  *kchunk = per * 32;
}

int gemm_chunk_splits(int K, int splits) {
  int used, per;
  chunk_plan(K, splits, &used, &per);
  return used;
}

// ------------------------------------------------------------------ wide tiles, fragment operands
// Many rows with both operands in the fragment layout of common.h.  A
// workgroup owns a 288 x BN output tile (BN = 128, or 64 for small products)
// and has four waves, one per SIMD, so at BN = 128 each may hold up to 512
// registers (at 64, two workgroups share a CU).  Wave w owns the 16-row blocks
// w, w + 4, ..., w + 16 across all BN columns (BN / 16 x 5 accumulators; the fifth block of
// waves 2 and 3 lies past the tile: it is computed on clamped rows and
// dropped).  Every row block belongs to one wave, so activation fragments go
// straight from global memory into registers (two register sets, issued two
// 64-wide K slices ahead) without touching LDS.  The weight slice, BN columns
// x 64 k = BN / 8 fragments of 1 KB, is shared by the four waves: each thread
// fetches BN / 32 of its 16-byte vectors into one of two register sets three
// slices ahead and writes them into one of two LDS buffers in fragment order,
// so every LDS read and write of a wave is a contiguous 1 KB.  One barrier per
// slice.  The MFMA takes the weight fragment as its first operand: a lane's
// accumulator then holds four consecutive columns of one row, and the
// epilogue stores 8 (bf16) or 16 (fp32) contiguous bytes per lane.  Slices past
// the end are fetched clamped and never computed; rows past M and columns past
// N are never stored.  (row, split) work items are numbered so that the
// workgroups of one XCD share a split's activation K range and whole weight
// panels.
struct FragP {
  const uint16_t* A;
  const uint16_t* W;
  int M, N, K, kchunk, nM, nN;
  Epilogue epi;
  float* ws;
};

constexpr int kFragBM = 288;

// The accumulator is pinned to the accumulation registers: with the builtin,
// the register allocator sometimes splits the 160 accumulators of k_gemm_af
// between the two register files and copies them back and forth every
// iteration.  The first k-step starts from a zero accumulator operand, so no
// register write precedes an MFMA; the caller inserts the wait states between
// the last MFMA and the first read of its results.
template <bool FIRST>
__device__ __forceinline__ void mfma16_acc(f32x4_t& c, bf16x8_t a, bf16x8_t b) {
  if (FIRST) asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=a"(c) : "v"(a), "v"(b));
  else asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_wait_states() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

__device__ __forceinline__ u32x2_t pack4_bf16(float a, float b, float c, float d) {
  return u32x2_t{pack_bf2(a, b), pack_bf2(c, d)};
}

template <int KIND, bool ODD, int BN>
__global__ __launch_bounds__(256, BN == 64 ? 2 : 1) void k_gemm_af(FragP p) {
  constexpr int RB = kFragBM / 16, TB = 5, NB = BN / 16, KS = 2, FR = NB * KS, WV = FR / 4;
  __shared__ u32x4_t sw[2][FR][64];
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int total = gridDim.x, L = blockIdx.x;
  const int q = (total % 8 == 0) ? (L % 8) * (total / 8) + L / 8 : L;
  const int ntile = p.nM * p.nN;
  const int split = q / ntile, tile = q - split * ntile;
  const int tm = tile % p.nM, tn = tile / p.nM;
  const int KSt = p.K >> 5;
  const int kb0 = split * (p.kchunk >> 5);
  const int nsl = max(0, min(p.kchunk, p.K - split * p.kchunk) >> 6);
  const int mbt = (p.M + 15) >> 4, nbt = p.N >> 4;

  // wave-uniform fragment bases (scalar registers) plus one per-lane byte offset
  const char* ab[TB];
#pragma unroll
  for (int i = 0; i < TB; ++i)
    ab[i] = (const char*)p.A + ((long)min(tm * RB + w + 4 * i, mbt - 1) * KSt + kb0) * 1024;
  const char* wb[WV];
#pragma unroll
  for (int i = 0; i < WV; ++i) {
    const int f = w + 4 * i, nb = f / KS, kk = f % KS;
    wb[i] = (const char*)p.W + ((long)min(tn * NB + nb, nbt - 1) * KSt + kb0 + kk) * 1024;
  }
  const uint32_t lo = lane * 16;
  auto soff = [&](int s) { return (uint32_t)min(s, max(nsl - 1, 0)) * (KS * 1024); };
  u32x4_t a0[TB][KS], a1[TB][KS], w0[WV], w1[WV];
  auto lda = [&](u32x4_t(&a)[TB][KS], int s) {
    const uint32_t o = soff(s) + lo;
#pragma unroll
    for (int i = 0; i < TB; ++i)
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) a[i][kk] = *(const u32x4_t*)(ab[i] + o + kk * 1024);
  };
  auto ldw = [&](u32x4_t(&r)[WV], int s) {
    const uint32_t o = soff(s) + lo;
#pragma unroll
    for (int i = 0; i < WV; ++i) r[i] = *(const u32x4_t*)(wb[i] + o);
  };
  auto stw = [&](const u32x4_t(&r)[WV], int buf) {
#pragma unroll
    for (int i = 0; i < WV; ++i) sw[buf][w + 4 * i][lane] = r[i];
  };
  f32x4_t acc[TB][NB];
  // MFMAs run weight fragment by weight fragment; as soon as fragment j has
  // served its five row blocks, the same k-step's successor is read into its
  // registers, so at most one k-step of fragments is live and each read has
  // the rest of the k-step to land.  The fences pin that order (left to
  // itself the compiler hoists every read and runs out of registers).
  auto compute = [&](const u32x4_t(&a)[TB][KS], int buf, auto first) {
    bf16x8_t b[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) b[j] = as_bf16x8(sw[buf][j * KS][lane]);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
#pragma unroll
      for (int j = 0; j < NB; ++j) {
#pragma unroll
        for (int i = 0; i < TB; ++i) {
          if (decltype(first)::value && kk == 0) mfma16_acc<true>(acc[i][j], b[j], as_bf16x8(a[i][kk]));
          else mfma16_acc<false>(acc[i][j], b[j], as_bf16x8(a[i][kk]));
        }
        if (kk + 1 < KS) b[j] = as_bf16x8(sw[buf][j * KS + kk + 1][lane]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  using First = std::integral_constant<bool, true>;
  using Next = std::integral_constant<bool, false>;

  // entering slice s (even): W(s) in LDS buffer 0, W(s+1) in w1, W(s+2) in w0, A(s) in a0, A(s+1) in a1
  ldw(w0, 0);
  ldw(w1, 1);
  lda(a0, 0);
  lda(a1, 1);
  stw(w0, 0);
  ldw(w0, 2);
  __syncthreads();
  // scheduling barriers keep each register set's reload behind its last use
  auto two_slices = [&](int s, auto first) {
    stw(w1, 1);
    __builtin_amdgcn_sched_barrier(0);
    ldw(w1, s + 3);
    compute(a0, 0, first);
    __builtin_amdgcn_sched_barrier(0);
    lda(a0, s + 2);
    __syncthreads();
    stw(w0, 0);
    __builtin_amdgcn_sched_barrier(0);
    ldw(w0, s + 4);
    if (ODD && s + 1 >= nsl) {  // odd slice count: the pair's second half adds nothing
#pragma unroll
      for (int i = 0; i < TB; ++i)
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) a1[i][kk] = u32x4_t{0, 0, 0, 0};
    }
    compute(a1, 1, Next{});
    __builtin_amdgcn_sched_barrier(0);
    lda(a1, s + 3);
    __syncthreads();
  };
  two_slices(0, First{});
  for (int s = 2; s < nsl; s += 2) two_slices(s, Next{});

  // the results are read below by VALU and memory instructions, which the
  // compiler does not know the MFMAs above have to finish for
  mfma_wait_states();
#pragma unroll
  for (int i = 0; i < TB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) asm volatile("" : "+a"(acc[i][j]));
  // epilogue: accumulator element e of lane l is row l % 16 and column (l / 16) * 4 + e of its block
  const int cq = (lane >> 4) * 4;
#pragma unroll
  for (int i = 0; i < TB; ++i) {
    const int rb = w + 4 * i;
    const int m = tm * kFragBM + rb * 16 + (lane & 15);
    if (rb >= RB || m >= p.M || KIND == EPI_QKV || KIND == EPI_CACHE) continue;
    if (KIND == EPI_GEGLU) {
#pragma unroll
      for (int j = 0; j < NB; j += 2) {
        const int n = tn * BN + j * 16;
        if (n >= p.N) break;  // N % 32 == 0: a gate block in range has its up block
        const int f = (n >> 1) + cq;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = gelu_erf(acc[i][j][e]) * acc[i][j + 1][e];
        const Epilogue& E = p.epi;
        if (E.out_f32) {
          *(f32x4_t*)((float*)E.out + (long)m * E.ldo + f) = f32x4_t{v[0], v[1], v[2], v[3]};
        } else {
          const long o = E.out_frag ? frag_idx(m, f, E.ldo) : (long)m * E.ldo + f;
          *(u32x2_t*)((bf16_t*)E.out + o) = pack4_bf16(v[0], v[1], v[2], v[3]);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int n = tn * BN + j * 16 + cq;
        if (n >= p.N) break;
        // copy out through VALU registers: storing the accumulator registers
        // directly lets the register allocator move accumulators out of the
        // accumulation registers, which costs copies in the main loop
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[e] = acc[i][j][e];
          asm volatile("" : "+v"(x[e]));
        }
        const f32x4_t v = f32x4_t{x[0], x[1], x[2], x[3]};
        if (KIND == EPI_PARTIAL || KIND == EPI_STORE) {
          // partials are an fp32 store into the split's [M][N] slab
          const bool f32 = KIND == EPI_PARTIAL || p.epi.out_f32;
          void* out = KIND == EPI_PARTIAL ? (void*)(p.ws + (long)split * p.M * p.N) : p.epi.out;
          const long o = (long)m * (KIND == EPI_PARTIAL ? p.N : p.epi.ldo) + n;
          if (f32) *(f32x4_t*)((float*)out + o) = v;
          else *(u32x2_t*)((bf16_t*)out + o) = pack4_bf16(v[0], v[1], v[2], v[3]);
        } else if (KIND == EPI_RESID) {
          f32x4_t* r = (f32x4_t*)(p.epi.resid + (long)m * p.epi.ldr + n);
          *r = *r + v;
        }
      }
    }
  }
  if (KIND == EPI_QKV || KIND == EPI_CACHE) {
    // element-wise scatters: a row block's accumulators go through this wave's
    // quarter of the (now idle) LDS so the store loop can stay rolled
    float* st = (float*)&sw[0][0][0] + w * (NB * 4 * 64);
#pragma unroll
    for (int i = 0; i < TB; ++i) {
      const int rb = w + 4 * i;
      const int m = tm * kFragBM + rb * 16 + (lane & 15);
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float x = acc[i][j][e];
          asm volatile("" : "+v"(x));
          st[(j * 4 + e) * 64 + lane] = x;
        }
      if (rb < RB && m < p.M) {
#pragma unroll 1
        for (int j = 0; j < NB; ++j) {
          const int n = tn * BN + j * 16 + cq;
          if (n >= p.N) break;
#pragma unroll 1
          for (int e = 0; e < 4; ++e) epi_store_t<KIND>(p.epi, m, n + e, st[(j * 4 + e) * 64 + lane]);
        }
      }
    }
  }
}

// The same 288 x 128 tile with eight waves, two per SIMD: wave w owns row
// blocks w, w + 8 (and w + 16 for waves 0 and 1), so SIMD s carries waves s and
// s + 4 with five or four row blocks between them, as the four-wave kernel.
// While one wave of a SIMD waits (on its loads, the LDS or the barrier) the
// other issues MFMAs.  Each wave holds at most 3 x 8 accumulators, so both fit
// the SIMD's registers; the weight slice's 16 fragments are staged by all 512
// threads, two vectors each.  GeGLU, partial-sum and plain store epilogues.
template <int TBW, int KIND, bool ODD>
__device__ __forceinline__ void af8_body(const FragP& p, u32x4_t (*sw)[16][64], int w, int lane, int tm, int tn,
                                         int split, int nsl, int kb0) {
  constexpr int RB = kFragBM / 16, NB = 8, KS = 2, BN = 128;
  const int KSt = p.K >> 5;
  const int mbt = (p.M + 15) >> 4, nbt = p.N >> 4;
  const char* ab[TBW];
#pragma unroll
  for (int i = 0; i < TBW; ++i)
    ab[i] = (const char*)p.A + ((long)min(tm * RB + w + 8 * i, mbt - 1) * KSt + kb0) * 1024;
  const char* wb[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int f = w + 8 * i, nb = f / KS, kk = f % KS;
    wb[i] = (const char*)p.W + ((long)min(tn * NB + nb, nbt - 1) * KSt + kb0 + kk) * 1024;
  }
  const uint32_t lo = lane * 16;
  auto soff = [&](int s) { return (uint32_t)min(s, max(nsl - 1, 0)) * (KS * 1024); };
  u32x4_t a0[TBW][KS], a1[TBW][KS], a2[TBW][KS], w0[2], w1[2];
  auto lda = [&](u32x4_t(&a)[TBW][KS], int s) {
    const uint32_t o = soff(s) + lo;
#pragma unroll
    for (int i = 0; i < TBW; ++i)
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) a[i][kk] = *(const u32x4_t*)(ab[i] + o + kk * 1024);
  };
  auto ldw = [&](u32x4_t(&r)[2], int s) {
    const uint32_t o = soff(s) + lo;
#pragma unroll
    for (int i = 0; i < 2; ++i) r[i] = *(const u32x4_t*)(wb[i] + o);
  };
  auto stw = [&](const u32x4_t(&r)[2], int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) sw[buf][w + 8 * i][lane] = r[i];
  };
  f32x4_t acc[TBW][NB];
  auto compute = [&](const u32x4_t(&a)[TBW][KS], int buf, auto first) {
    bf16x8_t b[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) b[j] = as_bf16x8(sw[buf][j * KS][lane]);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
#pragma unroll
      for (int j = 0; j < NB; ++j) {
#pragma unroll
        for (int i = 0; i < TBW; ++i) {
          if (decltype(first)::value && kk == 0) mfma16_acc<true>(acc[i][j], b[j], as_bf16x8(a[i][kk]));
          else mfma16_acc<false>(acc[i][j], b[j], as_bf16x8(a[i][kk]));
        }
        if (kk + 1 < KS) b[j] = as_bf16x8(sw[buf][j * KS + kk + 1][lane]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  using First = std::integral_constant<bool, true>;
  using Next = std::integral_constant<bool, false>;
  // Activation fragments rotate through three register sets (slice t in set
  // t % 3, fetched three slices ahead from L2); weight slices through two
  // register sets and two LDS buffers.
  ldw(w0, 0);
  ldw(w1, 1);
  lda(a0, 0);
  lda(a1, 1);
  lda(a2, 2);
  stw(w0, 0);
  ldw(w0, 2);
  __syncthreads();
  auto slice = [&](int t, u32x4_t(&wn)[2], u32x4_t(&a)[TBW][KS], auto first) {
    stw(wn, (t + 1) & 1);  // slice t + 1 into the buffer slice t - 1 used
    __builtin_amdgcn_sched_barrier(0);
    ldw(wn, t + 3);
    compute(a, t & 1, first);
    __builtin_amdgcn_sched_barrier(0);
    lda(a, t + 3);
    __syncthreads();
  };
  for (int s = 0; s < nsl; s += 6) {
    if (s == 0) slice(0, w1, a0, First{});
    else slice(s, w1, a0, Next{});
    if (s + 1 < nsl) slice(s + 1, w0, a1, Next{});
    if (s + 2 < nsl) slice(s + 2, w1, a2, Next{});
    if (s + 3 < nsl) slice(s + 3, w0, a0, Next{});
    if (s + 4 < nsl) slice(s + 4, w1, a1, Next{});
    if (s + 5 < nsl) slice(s + 5, w0, a2, Next{});
  }
  mfma_wait_states();
#pragma unroll
  for (int i = 0; i < TBW; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) asm volatile("" : "+a"(acc[i][j]));
  const int cq = (lane >> 4) * 4;
#pragma unroll
  for (int i = 0; i < TBW; ++i) {
    const int rb = w + 8 * i;
    const int m = tm * kFragBM + rb * 16 + (lane & 15);
    if (rb >= RB || m >= p.M) continue;
    if (KIND == EPI_GEGLU) {
#pragma unroll
      for (int j = 0; j < NB; j += 2) {
        const int n = tn * BN + j * 16;
        if (n >= p.N) break;
        const int f = (n >> 1) + cq;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = gelu_erf(acc[i][j][e]) * acc[i][j + 1][e];
        const Epilogue& E = p.epi;
        if (E.out_f32) {
          *(f32x4_t*)((float*)E.out + (long)m * E.ldo + f) = f32x4_t{v[0], v[1], v[2], v[3]};
        } else {
          const long o = E.out_frag ? frag_idx(m, f, E.ldo) : (long)m * E.ldo + f;
          *(u32x2_t*)((bf16_t*)E.out + o) = pack4_bf16(v[0], v[1], v[2], v[3]);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int n = tn * BN + j * 16 + cq;
        if (n >= p.N) break;
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[e] = acc[i][j][e];
          asm volatile("" : "+v"(x[e]));
        }
        const f32x4_t v = f32x4_t{x[0], x[1], x[2], x[3]};
        const bool f32 = KIND == EPI_PARTIAL || p.epi.out_f32;
        void* out = KIND == EPI_PARTIAL ? (void*)(p.ws + (long)split * p.M * p.N) : p.epi.out;
        const long o = (long)m * (KIND == EPI_PARTIAL ? p.N : p.epi.ldo) + n;
        if (f32) *(f32x4_t*)((float*)out + o) = v;
        else *(u32x2_t*)((bf16_t*)out + o) = pack4_bf16(v[0], v[1], v[2], v[3]);
      }
    }
  }
}

template <int KIND, bool ODD>
__global__ __launch_bounds__(512, 1) void k_gemm_af8(FragP p) {
  static_assert(KIND == EPI_GEGLU || KIND == EPI_PARTIAL || KIND == EPI_STORE, "epilogue kinds of the 8-wave kernel");
  __shared__ u32x4_t sw[2][16][64];
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int total = gridDim.x, L = blockIdx.x;
  const int q = (total % 8 == 0) ? (L % 8) * (total / 8) + L / 8 : L;
  const int ntile = p.nM * p.nN;
  const int split = q / ntile, tile = q - split * ntile;
  const int tm = tile % p.nM, tn = tile / p.nM;
  const int kb0 = split * (p.kchunk >> 5);
  const int nsl = max(0, min(p.kchunk, p.K - split * p.kchunk) >> 6);
  if (w < 2) af8_body<3, KIND, ODD>(p, sw, w, lane, tm, tn, split, nsl, kb0);
  else af8_body<2, KIND, ODD>(p, sw, w, lane, tm, tn, split, nsl, kb0);
}

// Row tiles over the whole K range, for the prefix's narrow products that
// finish in place at a few hundred rows (the fused QKV with its scatter, the
// O projection added into the residual).  With 288-row tiles such a product
// has 20-40 tiles, so it needs split-K partials to fill the chip, and the
// partials then cost a reduction kernel (QKV) or a norm reading every slab
// back (O).  Here a workgroup owns 96 x 32 outputs (six row blocks by two
// column blocks) over the whole K range: its eight waves take K / 8 each with
// three register sets of two k-steps (six k-steps of fragments in flight), the
// partial tiles meet once in LDS in wave order, and waves 0-5 finish one row
// block each: every output is stored once, by its owner.
constexpr int kRkMB = 6, kRkNB = 2;
constexpr int kRkSets = 3;
constexpr int kRkMaxRows = 320;  // above this the 288-row tiles with split-K win (more rows share each weight read)

template <int KIND, int PW>
__global__ __launch_bounds__(512) void k_gemm_rk(FragP p) {
  constexpr int MB = kRkMB, NB = kRkNB, G = 2, NG = PW / G;
  constexpr int NS = NG < kRkSets ? NG : kRkSets;  // register sets: groups of G k-steps in flight
  static_assert(PW % G == 0 && NG >= 1, "k-steps per wave");
  __shared__ float red[8][MB * NB * 4][64];  // [wave][row block, column block, element][lane]
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int tn = blockIdx.x, tm = blockIdx.y;
  const int KS = p.K >> 5, mbt = (p.M + 15) >> 4;
  const int sb = w * PW, nst = max(0, min(PW, KS - sb));  // this wave's k-steps
  const u32x4_t* Av = (const u32x4_t*)p.A + lane;
  const u32x4_t* Wv = (const u32x4_t*)p.W + lane;
  int arow[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) arow[i] = min(tm * MB + i, mbt - 1);  // clamped blocks: computed, never stored
  u32x4_t af[NS][G][MB], wf[NS][G][NB];
  auto load = [&](int set, int j) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int ks = min(sb + G * j + g, KS - 1);  // clamped; steps past the range are masked below
#pragma unroll
      for (int i = 0; i < MB; ++i) af[set][g][i] = Av[((long)arow[i] * KS + ks) * 64];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) wf[set][g][nb] = Wv[((long)(tn * NB + nb) * KS + ks) * 64];
    }
  };
  f32x4_t acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[i][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto comp = [&](int set, int j) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const bool on = G * j + g < nst;
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const u32x4_t a4 = on ? af[set][g][i] : u32x4_t{0, 0, 0, 0};
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[i][nb] = mfma16x16x32(as_bf16x8(a4), as_bf16x8(wf[set][g][nb]), acc[i][nb]);
      }
    }
  };
  // straight-line schedule (the loops unroll fully): group j in set j % NS,
  // refilled with group j + NS once multiplied
#pragma unroll
  for (int j = 0; j < NS; ++j) load(j, j);
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    comp(j % NS, j);
    if (j + NS < NG) load(j % NS, j + NS);
  }
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int e = 0; e < 4; ++e) red[w][(i * NB + nb) * 4 + e][lane] = acc[i][nb][e];
  __syncthreads();
  if (w >= MB) return;
  // wave w finishes row block w: the eight K ranges summed in wave order
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = (w * NB + nb) * 4 + e;
      float v = red[0][idx][lane];
#pragma unroll
      for (int ww = 1; ww < 8; ++ww) v += red[ww][idx][lane];
      const int m = (tm * MB + w) * 16 + grp * 4 + e, n = (tn * NB + nb) * 16 + col;
      if (m < p.M) epi_store_t<KIND>(p.epi, m, n, v);
    }
}

// K is cut into chunks of an even number of 64-wide slices (the kernel runs
// slices in pairs; only the last chunk may hold an odd count); `splits` <= 0
// asks for the count frag_per estimates fastest.
// Tile width: 64 columns for the small square products (two workgroups then
// share a CU, and the grid reaches the CU count with fewer K splits), 128 else.
// 64-column tiles (two workgroups per CU) for products of at most 2048-deep K
// and at most 2048 columns, and for wider ones that 128-column tiles would
// spread over fewer than 32 CUs (the 288-token prefix QKV: 20 tiles; with 64
// columns the whole prefix went from 2.38 to 2.31 ms); 128 columns otherwise.  (At 60-72 tiles, the dual-arm and batched QKV and cache
// projections, the two widths measured within noise of each other.)
static int frag_bn(int M, int N, int K) {
  if (K > 2048) return 128;
  if (N <= 2048) return 64;
  const int tiles128 = (M + kFragBM - 1) / kFragBM * ((N + 127) / 128);
  return tiles128 < 32 ? 64 : 128;
}

// K splits of a product on the 288-row tiles (`splits` <= 0: automatic): the
// count that minimises an estimate of the busiest CU's time, rounds of
// workgroups times the bytes each pulls through its CU, plus the partial slabs
// written and read back (about 5 TB/s) and, for a product that finishes in the
// GEMM (`kind` not EPI_PARTIAL), the reduction's launch (about 4 us; such
// products split at most four ways).  A CU pulls about 52 GB/s in the eight-wave
// kernel (128-column tiles with a GeGLU, partial-sum or plain store epilogue;
// the prefix gate/up GEMM's rate) and in the 64-column kernel, about 16 GB/s in
// the four-wave 128-column kernel that the scatter epilogues run on unsplit (the
// 800-row expert QKV took 55 us there against 26 us split four ways).  Ties go
// to fewer splits.  Returns 128-deep K pairs per chunk.
static int frag_per(int M, int N, int K, int splits, int bn, int kind) {
  const int pairs = (K / 64 + 1) / 2;
  if (splits > 0) {
    splits = std::max(1, std::min(splits, pairs));
    return (pairs + splits - 1) / splits;
  }
  const bool finishing = kind != EPI_PARTIAL;
  const int tiles = (M + kFragBM - 1) / kFragBM * ((N + bn - 1) / bn);
  double best = 0.0;
  int best_per = pairs;
  for (int per = pairs; per >= 1; --per) {
    const int used = (pairs + per - 1) / per;
    if (used > 16 || (finishing && used > 4)) break;
    const int k_run = used > 1 ? EPI_PARTIAL : kind;  // the epilogue the tile kernel runs
    const bool slow = bn == 128 && k_run != EPI_GEGLU && k_run != EPI_PARTIAL && k_run != EPI_STORE;
    const int rounds = (tiles * used + 255) / 256;
    double t = (double)rounds * (kFragBM + bn) * per * 128 * 2 / (slow ? 16e9 : 52e9);
    if (used > 1 || !finishing) t += (double)used * M * N * 8 / 5e12;
    if (used > 1 && finishing) t += 4e-6;
    if (per == pairs || t < best * 0.999) {
      best = t;
      best_per = per;
    }
  }
  return best_per;
}

int gemm_frag_splits(int M, int N, int K, int splits, int kind) {
  if (K < 64) return 1;
  const int per = frag_per(M, N, K, splits, frag_bn(M, N, K), kind);
  return ((K / 64 + 1) / 2 + per - 1) / per;
}

template <bool ODD, int BN>
static hipError_t launch_af(const FragP& p, int kind, dim3 grid, hipStream_t s) {
  switch (kind) {
    case EPI_STORE: hipLaunchKernelGGL((k_gemm_af<EPI_STORE, ODD, BN>), grid, dim3(256), 0, s, p); break;
    case EPI_GEGLU: hipLaunchKernelGGL((k_gemm_af<EPI_GEGLU, ODD, BN>), grid, dim3(256), 0, s, p); break;
    case EPI_PARTIAL: hipLaunchKernelGGL((k_gemm_af<EPI_PARTIAL, ODD, BN>), grid, dim3(256), 0, s, p); break;
    case EPI_QKV: hipLaunchKernelGGL((k_gemm_af<EPI_QKV, ODD, BN>), grid, dim3(256), 0, s, p); break;
    case EPI_CACHE: hipLaunchKernelGGL((k_gemm_af<EPI_CACHE, ODD, BN>), grid, dim3(256), 0, s, p); break;
    case EPI_RESID: hipLaunchKernelGGL((k_gemm_af<EPI_RESID, ODD, BN>), grid, dim3(256), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool ODD>
static hipError_t launch_af8(const FragP& p, int kind, dim3 grid, hipStream_t s) {
  switch (kind) {
    case EPI_STORE: hipLaunchKernelGGL((k_gemm_af8<EPI_STORE, ODD>), grid, dim3(512), 0, s, p); break;
    case EPI_GEGLU: hipLaunchKernelGGL((k_gemm_af8<EPI_GEGLU, ODD>), grid, dim3(512), 0, s, p); break;
    case EPI_PARTIAL: hipLaunchKernelGGL((k_gemm_af8<EPI_PARTIAL, ODD>), grid, dim3(512), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

bool gemm_frag_rowtile(int M, int N, int K, int kind) {
  return (kind == EPI_QKV || kind == EPI_RESID) && M > 64 && M <= kRkMaxRows && N % (16 * kRkNB) == 0 && K % 32 == 0 &&
         K <= 8 * 8 * 32;
}

hipError_t gemm_frag(const uint16_t* Af, const uint16_t* Wf, int M, int N, int K, const Epilogue& epi, int splits,
                     float* ws, hipStream_t s) {
  if (M <= 0 || N <= 0 || K <= 0) return hipSuccess;
  if (K % 64 || N % 32) return hipErrorInvalidValue;
  const int kind0 = epi.kind;
  if ((kind0 == EPI_STORE || kind0 == EPI_GEGLU) && epi.ldo % 4) return hipErrorInvalidValue;
  if (kind0 == EPI_RESID && epi.ldr % 4) return hipErrorInvalidValue;
  if (epi.out_frag && kind0 != EPI_GEGLU && kind0 != EPI_CACHE) return hipErrorInvalidValue;
  if (epi.out_frag && epi.out_f32) return hipErrorInvalidValue;
  if (splits <= 0 && gemm_frag_rowtile(M, N, K, kind0)) {
    FragP p{Af, Wf, M, N, K, 0, 0, 0, epi, ws};
    const dim3 grid(N / (16 * kRkNB), (M + 16 * kRkMB - 1) / (16 * kRkMB));
    const int pw = (K / 32 + 7) / 8;  // k-steps per wave
#define VLA_RK(KIND, PW) hipLaunchKernelGGL((k_gemm_rk<KIND, PW>), grid, dim3(512), 0, s, p)
    if (kind0 == EPI_QKV) {
      if (pw <= 2) VLA_RK(EPI_QKV, 2); else if (pw <= 4) VLA_RK(EPI_QKV, 4); else VLA_RK(EPI_QKV, 8);
    } else {
      if (pw <= 2) VLA_RK(EPI_RESID, 2); else if (pw <= 4) VLA_RK(EPI_RESID, 4); else VLA_RK(EPI_RESID, 8);
    }
#undef VLA_RK
    return hipGetLastError();
  }
  const int bn = frag_bn(M, N, K);
  int per = frag_per(M, N, K, splits, bn, kind0);
  splits = ((K / 64 + 1) / 2 + per - 1) / per;
  if ((splits > 1 || kind0 == EPI_PARTIAL) && !ws) return hipErrorInvalidValue;
  FragP p{Af, Wf, M, N, K, 0, 0, 0, epi, ws};
  p.nM = (M + kFragBM - 1) / kFragBM;
  p.nN = (N + bn - 1) / bn;
  p.kchunk = per * 128;
  const dim3 grid(p.nM * p.nN * splits);
  const int kind = splits > 1 ? EPI_PARTIAL : kind0;
  const bool odd = (K / 64) % 2;
  hipError_t err;
  if (bn == 128 && (kind == EPI_GEGLU || kind == EPI_PARTIAL || kind == EPI_STORE)) {
    err = odd ? launch_af8<true>(p, kind, grid, s) : launch_af8<false>(p, kind, grid, s);  // eight waves
  } else {
    err = bn == 64 ? (odd ? launch_af<true, 64>(p, kind, grid, s) : launch_af<false, 64>(p, kind, grid, s))
                   : (odd ? launch_af<true, 128>(p, kind, grid, s) : launch_af<false, 128>(p, kind, grid, s));
  }
  if (err != hipSuccess) return err;
  if (splits > 1 && kind0 != EPI_PARTIAL) {
    const long total = (long)M * N / 4;
    const int blocks = (int)std::min<long>((total + 255) / 256, 4096);
    hipLaunchKernelGGL(k_splitk_reduce, dim3(blocks), dim3(256), 0, s, (const float*)ws, splits, M, N, epi);
    err = hipGetLastError();
  }
  return err;
}

// ------------------------------------------------------------------ chunk rows, fragment layout
// Activations of at most 64 rows with both operands in the fragment layout of
// common.h.  A workgroup owns 16 * NB columns of every row block (or, split by
// rows, of one row block), its four waves split the K
// range (at most kChunkSteps k-steps each, issued at once: one memory round
// trip covers the slice) and their partial tiles are summed through LDS in
// wave order.  Every load of a wave is one contiguous 1 KB fragment: a weight
// fragment per 16 columns and k-step, an activation fragment per 16 rows and
// k-step.  MB is 1, 2 or 4 row blocks, the fewest that cover M; the activation
// buffer holds MB whole blocks, and rows past M are computed but never stored.
struct ChunkP {
  const uint16_t* A;
  const uint16_t* W;
  int M, N, K, kchunk;
  Epilogue epi;
  float* ws;
  Prefetch pf;  // read by grid layers z >= 1, if any
  int rsplit;   // 1: one 16-row block per workgroup (grid y), K not split
};

template <int NB, int MB, int KIND, int SPW, bool RS>
__global__ __launch_bounds__(256) void k_chunk(ChunkP p) {
  __shared__ float red[4][MB * NB * 4][64];  // [wave][row block, column block, element][lane]
  __shared__ float rsp[4][64];               // RS: each wave's partial sum of squares of each row
  if (prefetch_layer(p.pf)) return;
  // RS: the partial sums of squares are laid out [x][row][S] (x the producer's
  // XCD, S = nss / 8 column groups each); lane l of wave w takes row l's of
  // XCDs 2w and 2w + 1 (S consecutive floats each, so a wave's loads cover
  // whole lines).  They go out with the kernel's first loads and are summed
  // after its MFMAs.
  f32x4_t ssv[2][2];
  if (RS) {
    const int S = p.epi.nss >> 3;
#pragma unroll
    for (int xi = 0; xi < 2; ++xi) {
      const float* b = p.epi.rss + ((long)(2 * ((int)threadIdx.x >> 6) + xi) * 64 + (threadIdx.x & 63)) * S;
      if (S >= 4) {
        ssv[xi][0] = *(const f32x4_t*)b;
        ssv[xi][1] = S == 8 ? *(const f32x4_t*)(b + 4) : f32x4_t{0.f, 0.f, 0.f, 0.f};
      } else {
        ssv[xi][0] = f32x4_t{b[0], S == 2 ? b[1] : 0.f, 0.f, 0.f};
        ssv[xi][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
  }
  // visible keys (scores), requested with the operands
  const int nkey = KIND == EPI_SCORES ? (p.epi.klen ? min(uniform_ld(p.epi.klen, 0), p.epi.npre) : p.epi.npre) : 0;
  // column group, K chunk (or, split by rows, the workgroup's row block)
  const int bx = blockIdx.x, by = p.rsplit ? 0 : blockIdx.y, rb0 = p.rsplit ? blockIdx.y : 0;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int nb0 = bx * NB;  // first 16-column block of the workgroup
  const int KS = p.K >> 5;  // k-steps (fragments per 16-row block)
  const int sb = (by * p.kchunk + w * (p.kchunk >> 2)) >> 5;
  const int nsteps = max(0, min(KS - sb, p.kchunk >> 7));
  const u32x4_t* Wv = (const u32x4_t*)p.W + lane;
  const u32x4_t* Av = (const u32x4_t*)p.A + (long)rb0 * KS * 64 + lane;

  u32x4_t wv[SPW][NB], av[SPW][MB];
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
    const int ks = min(sb + s, KS - 1);  // clamped; steps past the range are masked below
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) wv[s][nb] = Wv[((long)(nb0 + nb) * KS + ks) * 64];
#pragma unroll
    for (int rb = 0; rb < MB; ++rb) av[s][rb] = Av[((long)rb * KS + ks) * 64];
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
#pragma unroll
  for (int rb = 0; rb < MB; ++rb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int e = 0; e < 4; ++e) red[w][(rb * NB + nb) * 4 + e][lane] = acc[rb][nb][e];
  if (RS) {
    float t = 0.f;
#pragma unroll
    for (int xi = 0; xi < 2; ++xi)
#pragma unroll
      for (int v = 0; v < 2; ++v) t += (ssv[xi][v][0] + ssv[xi][v][1]) + (ssv[xi][v][2] + ssv[xi][v][3]);
    rsp[w][lane] = t;
  }
  __syncthreads();

  // wave w finishes row block w: the four K ranges summed in wave order, then the epilogue
  const int rb = w;
  if (rb >= MB) return;
  const int row0 = (rb0 + rb) * 16;
  float v[NB][4];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = (rb * NB + nb) * 4 + e;
      v[nb][e] = red[0][idx][lane] + red[1][idx][lane] + red[2][idx][lane] + red[3][idx][lane];
    }
  if (KIND == EPI_SCORES) {
    // the workgroup's 32 columns are keys t0 .. t0 + 31 of one head: keys past
    // the visible count are masked, then per row the block max r (16-lane DPP
    // reductions, every lane of a row ends with the same bits) and the weights
    // 2^(s - r) with their sum
    const int c0 = bx * 32, t0 = c0 % p.epi.npad, nblk = p.N >> 5;
    const bool vis0 = t0 + col < nkey, vis1 = t0 + 16 + col < nkey;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = row0 + grp * 4 + e;
      float a = v[0][e], b = v[NB - 1][e];
      if (RS) {
        const float r = 1.0f / sqrtf(((rsp[0][m] + rsp[1][m]) + (rsp[2][m] + rsp[3][m])) / (float)p.epi.rdim + p.epi.reps);
        a *= r;
        b *= r;
      }
      a = vis0 ? a : -INFINITY;
      b = vis1 ? b : -INFINITY;
      float mx = fmaxf(a, b);
      mx = fmaxf(mx, dpp_mov<0xB1>(mx));
      mx = fmaxf(mx, dpp_mov<0x4E>(mx));
      mx = fmaxf(mx, dpp_mov<0x141>(mx));
      mx = fmaxf(mx, dpp_mov<0x140>(mx));
      const float ref = mx == -INFINITY ? 0.f : mx;  // a fully masked block: weights 0, max -inf
      a = fast_exp2(a - ref);
      b = fast_exp2(b - ref);
      float l = a + b;
      l += dpp_mov<0xB1>(l);
      l += dpp_mov<0x4E>(l);
      l += dpp_mov<0x141>(l);
      l += dpp_mov<0x140>(l);
      if (m < p.M) {
        bf16_t* o = (bf16_t*)p.epi.out;
        o[frag_idx(m, c0 + col, p.epi.ldo)] = f2bf(a);
        o[frag_idx(m, c0 + 16 + col, p.epi.ldo)] = f2bf(b);
        if (col == 0) *(float2*)(p.epi.stats + 2 * ((long)m * nblk + bx)) = make_float2(mx, l);
      }
    }
    return;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int m = row0 + grp * 4 + e;
    if (m >= p.M) continue;
    if (RS) {
      const float r = 1.0f / sqrtf(((rsp[0][m] + rsp[1][m]) + (rsp[2][m] + rsp[3][m])) / (float)p.epi.rdim + p.epi.reps);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) v[nb][e] *= r;
    }
    if (KIND == EPI_GEGLU) {
      epi_geglu(p.epi, m, (nb0 >> 1) * 16 + col, v[0][e], v[NB - 1][e]);
      continue;
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int n = (nb0 + nb) * 16 + col;
      if (KIND == EPI_PARTIAL) p.ws[((long)by * p.M + m) * p.N + n] = v[nb][e];
      else epi_store_t<KIND>(p.epi, m, n, v[nb][e]);
    }
  }
}

template <int MB, int SPW>
static hipError_t launch_chunk_spw(const ChunkP& p, int kind, dim3 grid, hipStream_t s) {
  const bool rs = p.epi.rss != nullptr;  // row scales: the finishing kinds only
  switch (kind) {
    case EPI_GEGLU:
      if (rs) hipLaunchKernelGGL((k_chunk<2, MB, EPI_GEGLU, SPW, true>), grid, dim3(256), 0, s, p);
      else hipLaunchKernelGGL((k_chunk<2, MB, EPI_GEGLU, SPW, false>), grid, dim3(256), 0, s, p);
      break;
    case EPI_STORE:
      if (rs) hipLaunchKernelGGL((k_chunk<1, MB, EPI_STORE, SPW, true>), grid, dim3(256), 0, s, p);
      else hipLaunchKernelGGL((k_chunk<1, MB, EPI_STORE, SPW, false>), grid, dim3(256), 0, s, p);
      break;
    case EPI_QKV:
      if (rs) hipLaunchKernelGGL((k_chunk<1, MB, EPI_QKV, SPW, true>), grid, dim3(256), 0, s, p);
      else hipLaunchKernelGGL((k_chunk<1, MB, EPI_QKV, SPW, false>), grid, dim3(256), 0, s, p);
      break;
    case EPI_CACHE: hipLaunchKernelGGL((k_chunk<1, MB, EPI_CACHE, SPW, false>), grid, dim3(256), 0, s, p); break;
    case EPI_SCORES:
      if (rs) hipLaunchKernelGGL((k_chunk<2, MB, EPI_SCORES, SPW, true>), grid, dim3(256), 0, s, p);
      else hipLaunchKernelGGL((k_chunk<2, MB, EPI_SCORES, SPW, false>), grid, dim3(256), 0, s, p);
      break;
    case EPI_PARTIAL: hipLaunchKernelGGL((k_chunk<1, MB, EPI_PARTIAL, SPW, false>), grid, dim3(256), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// A wave loads SPW k-steps at once: the smallest of 2, 4 and 8 that covers its
// quarter of the workgroup's K chunk, so no wave fetches fragments it would
// mask off (a fixed 8 made the O projections, four k-steps per wave, fetch
// twice their bytes).
template <int MB>
static hipError_t launch_chunk_mb(const ChunkP& p, int kind, dim3 grid, hipStream_t s) {
  const int steps = p.kchunk >> 7;
  if (steps <= 2) return launch_chunk_spw<MB, 2>(p, kind, grid, s);
  if (steps <= 4) return launch_chunk_spw<MB, 4>(p, kind, grid, s);
  return launch_chunk_spw<MB, kChunkSteps>(p, kind, grid, s);
}

hipError_t gemm_chunk(const uint16_t* Af, const uint16_t* Wf, int M, int N, int K, const Epilogue& epi, int splits,
                      float* ws, hipStream_t s, const Prefetch* prefetch) {
  if (M <= 0 || N <= 0 || K <= 0) return hipSuccess;
  if (M > 64 || K % 32 || N % 32) return hipErrorInvalidValue;
  if (epi.kind != EPI_STORE && epi.kind != EPI_PARTIAL && epi.kind != EPI_GEGLU && epi.kind != EPI_QKV &&
      epi.kind != EPI_CACHE && epi.kind != EPI_SCORES)
    return hipErrorInvalidValue;
  int used, per;
  chunk_plan(K, splits, &used, &per);
  if (used > 1 && !ws) return hipErrorInvalidValue;
  // scores: whole 32-key blocks of whole heads, one K chunk, bf16 fragment-layout weights out
  if (epi.kind == EPI_SCORES &&
      (used > 1 || !epi.out || !epi.stats || epi.ldo != N || epi.npad <= 0 || epi.npad % 32 || N % epi.npad ||
       epi.npre <= 0 || epi.npre > epi.npad || ((uintptr_t)epi.stats & 7)))
    return hipErrorInvalidValue;
  // row scales apply to one K chunk's finished sums (no partials), at most 64 partials a row
  if (epi.rss && (used > 1 || epi.kind == EPI_PARTIAL || epi.kind == EPI_CACHE ||
                  (epi.nss != 8 && epi.nss != 16 && epi.nss != 32 && epi.nss != 64) || epi.rdim <= 0 ||
                  ((uintptr_t)epi.rss & 15)))
    return hipErrorInvalidValue;
  const Prefetch pf = prefetch ? *prefetch : Prefetch{};
  if (pf.blocks < 0 || pf.blocks > 1024 || (pf.blocks && !pf.sink)) return hipErrorInvalidValue;
  const bool reduce = used > 1 && epi.kind != EPI_PARTIAL;
  const int nb = (epi.kind == EPI_GEGLU || epi.kind == EPI_SCORES) && !reduce ? 2 : 1;
  const int kind = reduce ? EPI_PARTIAL : epi.kind;
  const int mb = (M + 15) / 16;
  // One 16-column block per workgroup (plain and QKV stores): with all rows
  // each workgroup pulls four times as many activation bytes as weight bytes,
  // so one row block per workgroup (four times the workgroups, each weight
  // slice read once per row block, from L2) moves far fewer bytes per CU:
  // cross query 5.7 -> about 4.8 us at 50 rows.  Two-column GeGLU workgroups
  // already fill the chip and would read their weights four times over.
  const int rsplit = used == 1 && mb > 1 && (kind == EPI_STORE || kind == EPI_QKV || kind == EPI_SCORES) ? 1 : 0;
  ChunkP p{Af, Wf, M, N, K, per * 32, epi, ws, pf, rsplit};
  const int gy = rsplit ? mb : used;
  const dim3 grid(N / (16 * nb), gy, prefetch_depth(N / (16 * nb) * gy, pf.blocks));
  hipError_t err = mb == 1 || rsplit ? launch_chunk_mb<1>(p, kind, grid, s)
                 : mb == 2           ? launch_chunk_mb<2>(p, kind, grid, s)
                                     : launch_chunk_mb<4>(p, kind, grid, s);
  if (err != hipSuccess) return err;
  if (reduce) {
    const long tot = (long)M * N / 4;
    const int blocks = (int)std::min<long>((tot + 255) / 256, 4096);
    hipLaunchKernelGGL(k_splitk_reduce, dim3(blocks), dim3(256), 0, s, (const float*)ws, used, M, N, epi);
    err = hipGetLastError();
  }
  return err;
}

// ------------------------------------------------------------------ residual-updating rows
// gemm_chunk_resnorm: a workgroup owns one 16-row block x 16 columns over the
// whole K range; its eight waves take K / 8 each (all of a wave's fragments
// requested at once, two accumulators so consecutive MFMAs do not wait on each
// other), summed through LDS in wave order.  Wave 0 then adds the residual,
// writes it back, and writes the next product's unnormalised input and the
// row's partial sum of squares over its 16 columns.
struct ResP {
  const uint16_t* A;
  const uint16_t* W;
  int M, N, K;
  float* h;
  int ldh;
  const float* gain;
  uint16_t* xb;
  float* ss;
  Prefetch pf;
};

constexpr bool kResXcdMajor = true;

// The end of a residual-updating product of one 16 x 16 output block: the
// eight waves' partial sums (acc) meet in LDS in wave order, then wave 0 adds
// the residual values (hold) and writes the new residual and, with a gain
// (g1 = 1 + gain[n]; hold and g1 requested with the operands), the next
// product's unnormalised input and the block's partial sums of squares.  p by
// value: its fields stay in scalar registers across the stores.
__device__ __forceinline__ void res_finish(const ResP p, const f32x4_t (&acc)[2], const float (&hold)[4], float g1,
                                           float (*red)[4][64], int w, int lane, int n, int rb) {
  const int col = lane & 15, grp = lane >> 4;
  // where this block's sums of squares go, [x][row][column group of x] (read from the dispatch before the stores)
  const int ss_x = ((int)blockIdx.x & 7) * 64, ss_s = (int)(gridDim.x >> 3), ss_g = (int)(blockIdx.x >> 3);
#pragma unroll
  for (int e = 0; e < 4; ++e) red[w][e][lane] = acc[0][e] + acc[1][e];
  __syncthreads();
  if (w) return;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float v = red[0][e][lane];
#pragma unroll
    for (int ww = 1; ww < 8; ++ww) v += red[ww][e][lane];
    const int m = rb * 16 + grp * 4 + e;
    const float x = hold[e] + v;
    if (m < p.M) p.h[(long)m * p.ldh + n] = x;
    if (p.gain) {
      // sum of x^2 over the 16 columns (the 16 lanes of this lane's row of the
      // wave; every lane ends with the same bits)
      float q = x * x;
      q += dpp_mov<0xB1>(q);
      q += dpp_mov<0x4E>(q);
      q += dpp_mov<0x141>(q);
      q += dpp_mov<0x140>(q);
      if (m < p.M) {
        p.xb[frag_idx(m, n, p.N)] = f2bf(x * g1);
        if (col == 0) p.ss[(ss_x + m) * ss_s + ss_g] = q;
      }
    }
  }
}



template <int SPW>
__global__ __launch_bounds__(512) void k_chunk_res(ResP p) {
  __shared__ float red[8][4][64];
  if (prefetch_layer(p.pf)) return;
  // column block: with kResXcdMajor the blocks of one XCD (linear id % 8) are
  // adjacent, so the residual's and the input's lines are written by one L2
  const int bx = kResXcdMajor && !(gridDim.x & 7) ? (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3) : blockIdx.x;
  const int rb = blockIdx.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int KS = p.K >> 5, sb = w * SPW;
  const int nsteps = max(0, min(SPW, KS - sb));  // the last waves may hold fewer k-steps, or none
  const int n = bx * 16 + col;
  const u32x4_t* Wv = (const u32x4_t*)p.W + lane;
  const u32x4_t* Av = (const u32x4_t*)p.A + lane;
  u32x4_t wv[SPW], av[SPW];
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
    const int ks = min(sb + s, KS - 1);  // clamped; steps past the range are masked below
    wv[s] = Wv[((long)bx * KS + ks) * 64];
    av[s] = Av[((long)rb * KS + ks) * 64];
  }
  // the residual values this block updates, requested with the fragments
  float hold[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) hold[e] = p.h[(long)min(rb * 16 + grp * 4 + e, p.M - 1) * p.ldh + n];
  const float g1 = p.gain ? 1.0f + p.gain[n] : 0.f;
  // keep every load ahead of the first MFMA (the scheduler would otherwise
  // interleave them, a few in flight at a time)
  __builtin_amdgcn_sched_barrier(0);
  f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
    const u32x4_t a4 = s < nsteps ? av[s] : u32x4_t{0, 0, 0, 0};
    acc[s & 1] = mfma16x16x32(as_bf16x8(a4), as_bf16x8(wv[s]), acc[s & 1]);
  }
  res_finish(p, acc, hold, g1, red, w, lane, n, rb);
}

size_t gemm_chunk_resnorm_group_bytes(int N, int K) {
  const int gx = N / 16;
  if (N % 16 || gx % 8) return 0;
  const size_t g = (size_t)16 * K * 2 * (kResXcdMajor ? gx / 8 : 1);
  return g & (g - 1) ? 0 : g;
}

hipError_t gemm_chunk_resnorm(const uint16_t* Af, const uint16_t* Wf, int M, int N, int K, float* h, int ldh,
                              const float* gain, uint16_t* xb, float* ss, hipStream_t s, const Prefetch* prefetch) {
  if (M <= 0 || N <= 0 || K <= 0) return hipSuccess;
  if (M > 64 || N % 128 || N > 1024 || K % 32 || K > 4096 || !h || (gain && (!xb || !ss))) return hipErrorInvalidValue;
  const Prefetch pf = prefetch ? *prefetch : Prefetch{};
  if (pf.blocks < 0 || pf.blocks > 1024 || (pf.blocks && !pf.sink)) return hipErrorInvalidValue;
  ResP p{Af, Wf, M, N, K, h, ldh, gain, xb, ss, pf};
  const int rbs = (M + 15) / 16, wgs = N / 16 * rbs;
  const dim3 grid(N / 16, rbs, prefetch_depth(wgs, pf.blocks));
  // k-steps per wave: the fewest of 1, 2, 4, 8, 16 that cover an eighth of K
  const int spw = (K / 32 + 7) / 8;
  if (spw <= 1) hipLaunchKernelGGL(k_chunk_res<1>, grid, dim3(512), 0, s, p);
  else if (spw <= 2) hipLaunchKernelGGL(k_chunk_res<2>, grid, dim3(512), 0, s, p);
  else if (spw <= 4) hipLaunchKernelGGL(k_chunk_res<4>, grid, dim3(512), 0, s, p);
  else if (spw <= 8) hipLaunchKernelGGL(k_chunk_res<8>, grid, dim3(512), 0, s, p);
  else hipLaunchKernelGGL(k_chunk_res<16>, grid, dim3(512), 0, s, p);
  return hipGetLastError();
}

// ------------------------------------------------------------------ absorbed cross attention: residual update
// k_chunk_probres: k_chunk_res with A = the scores kernel's block weights
// 2^(s - r) (K = heads x padded keys, one k-step per 32-key block).  Each
// k-step's product goes to its own accumulator; thread (row, head) < 16 x heads
// combines the head's block statistics into the scale 2^(r - R) / L of each
// block (R the head's max, L its weight sum), and a wave adds its k-steps'
// products scaled by their blocks' factors, so each head's weights are
// normalised before the heads are summed.  The statistics are requested first,
// so the scales are formed while the operands are still in flight.
constexpr int kProbMaxKS = 128, kProbMaxBph = 16;

template <int SPW>
__global__ __launch_bounds__(512) void k_chunk_probres(ResP p, const float* stats, int bph) {
  __shared__ float red[8][4][64];
  __shared__ __attribute__((aligned(16))) float cs[kProbMaxKS][16];  // [k-step][row] scale
  if (prefetch_layer(p.pf)) return;
  const int bx = kResXcdMajor && !(gridDim.x & 7) ? (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3) : blockIdx.x;
  const int rb = blockIdx.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int KS = p.K >> 5, sb = w * SPW;
  const int nsteps = max(0, min(SPW, KS - sb));
  const int n = bx * 16 + col;
  // this thread's (row, head): the head's block statistics
  const int heads = KS / bph;
  const int sr = threadIdx.x & 15, sh = min((int)threadIdx.x >> 4, heads - 1);
  const float2* sp = (const float2*)stats + (long)(rb * 16 + sr) * KS + sh * bph;
  float2 st[kProbMaxBph];
#pragma unroll
  for (int i = 0; i < kProbMaxBph; ++i) st[i] = sp[min(i, bph - 1)];
  const u32x4_t* Wv = (const u32x4_t*)p.W + lane;
  const u32x4_t* Av = (const u32x4_t*)p.A + lane;
  u32x4_t wv[SPW], av[SPW];
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
    const int ks = min(sb + s, KS - 1);  // clamped; steps past the range are masked below
    wv[s] = Wv[((long)bx * KS + ks) * 64];
    av[s] = Av[((long)rb * KS + ks) * 64];
  }
  float hold[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) hold[e] = p.h[(long)min(rb * 16 + grp * 4 + e, p.M - 1) * p.ldh + n];
  const float g1 = p.gain ? 1.0f + p.gain[n] : 0.f;
  __builtin_amdgcn_sched_barrier(0);
  if ((int)threadIdx.x < 16 * heads) {
    float R = -INFINITY;
#pragma unroll
    for (int i = 0; i < kProbMaxBph; ++i)
      if (i < bph) R = fmaxf(R, st[i].x);
    float L = 0.f;
#pragma unroll
    for (int i = 0; i < kProbMaxBph; ++i)
      if (i < bph) L += st[i].y * fast_exp2(st[i].x - R);
    const float inv = L > 0.f ? 1.0f / L : 0.f;  // rows past M: zero statistics, zero scales
#pragma unroll
    for (int i = 0; i < kProbMaxBph; ++i)
      if (i < bph) cs[sh * bph + i][sr] = fast_exp2(st[i].x - R) * inv;
  }
  f32x4_t pr[SPW];
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
    const u32x4_t a4 = s < nsteps ? av[s] : u32x4_t{0, 0, 0, 0};
    pr[s] = mfma16x16x32(as_bf16x8(a4), as_bf16x8(wv[s]), f32x4_t{0.f, 0.f, 0.f, 0.f});
  }
  __syncthreads();
  f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
    if (s < nsteps) {
      const f32x4_t c = *(const f32x4_t*)&cs[sb + s][grp * 4];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[s & 1][e] = fmaf(c[e], pr[s][e], acc[s & 1][e]);
    }
  }
  res_finish(p, acc, hold, g1, red, w, lane, n, rb);
}

hipError_t gemm_chunk_probres(const uint16_t* pw, const float* stats, int bph, const uint16_t* Wf, int M, int N,
                              int K, float* h, int ldh, const float* gain, uint16_t* xb, float* ss, hipStream_t s,
                              const Prefetch* prefetch) {
  if (M <= 0 || N <= 0 || K <= 0) return hipSuccess;
  const int KS = K / 32;
  if (M > 64 || N % 128 || N > 1024 || K % 32 || KS > kProbMaxKS || !h || !stats || (gain && (!xb || !ss)) ||
      bph <= 0 || bph > kProbMaxBph || KS % bph || KS / bph > 32 || ((uintptr_t)stats & 7))
    return hipErrorInvalidValue;
  const Prefetch pf = prefetch ? *prefetch : Prefetch{};
  if (pf.blocks < 0 || pf.blocks > 1024 || (pf.blocks && !pf.sink)) return hipErrorInvalidValue;
  ResP p{pw, Wf, M, N, K, h, ldh, gain, xb, ss, pf};
  const int rbs = (M + 15) / 16, wgs = N / 16 * rbs;
  const dim3 grid(N / 16, rbs, prefetch_depth(wgs, pf.blocks));
  // k-steps per wave: the fewest of these that cover an eighth of K
  const int spw = (KS + 7) / 8;
  if (spw <= 1) hipLaunchKernelGGL(k_chunk_probres<1>, grid, dim3(512), 0, s, p, stats, bph);
  else if (spw <= 2) hipLaunchKernelGGL(k_chunk_probres<2>, grid, dim3(512), 0, s, p, stats, bph);
  else if (spw <= 4) hipLaunchKernelGGL(k_chunk_probres<4>, grid, dim3(512), 0, s, p, stats, bph);
  else if (spw <= 8) hipLaunchKernelGGL(k_chunk_probres<8>, grid, dim3(512), 0, s, p, stats, bph);
  else if (spw <= 9) hipLaunchKernelGGL(k_chunk_probres<9>, grid, dim3(512), 0, s, p, stats, bph);
  else if (spw <= 10) hipLaunchKernelGGL(k_chunk_probres<10>, grid, dim3(512), 0, s, p, stats, bph);
  else if (spw <= 12) hipLaunchKernelGGL(k_chunk_probres<12>, grid, dim3(512), 0, s, p, stats, bph);
  else hipLaunchKernelGGL(k_chunk_probres<16>, grid, dim3(512), 0, s, p, stats, bph);
  return hipGetLastError();
}

size_t gemm_chunk_group_bytes(int M, int N, int K, int kind, int splits) {
  if (M > 64 || K % 32 || N % 32) return 0;
  int used, per;
  chunk_plan(K, splits, &used, &per);
  const int nb = (kind == EPI_GEGLU || kind == EPI_SCORES) && used == 1 ? 2 : 1;
  const int gx = N / (16 * nb);
  return gx % 8 ? 0 : (size_t)nb * 16 * K * 2;
}

// row-major [N][K] -> fragment layout, one 16-byte vector (8 k) per thread
__global__ void k_frag_pack(const u32x4_t* src, int N, int K, uint16_t* dst) {
  const long vecs = (long)N * (K / 8);
  for (long v = blockIdx.x * (long)blockDim.x + threadIdx.x; v < vecs; v += (long)gridDim.x * blockDim.x) {
    const int n = (int)(v / (K / 8)), k = (int)(v % (K / 8)) * 8;
    *(u32x4_t*)(dst + frag_idx(n, k, K)) = src[v];
  }
}

// row-major [R][C] -> fragment layout of the transpose [C][R]: a thread gathers
// the 8 source rows of one output vector (a one-time weight transform)
__global__ void k_frag_pack_t(const uint16_t* src, int R, int C, uint16_t* dst) {
  const long vecs = (long)C * (R / 8);
  for (long v = blockIdx.x * (long)blockDim.x + threadIdx.x; v < vecs; v += (long)gridDim.x * blockDim.x) {
    const int n = (int)(v % C), k = (int)(v / C) * 8;  // consecutive threads: consecutive source columns
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (uint32_t)src[(long)(k + 2 * i) * C + n] | ((uint32_t)src[(long)(k + 2 * i + 1) * C + n] << 16);
    *(u32x4_t*)(dst + frag_idx(n, k, R)) = u32x4_t{w[0], w[1], w[2], w[3]};
  }
}

hipError_t frag_pack_t(const uint16_t* src, int R, int C, uint16_t* dst, hipStream_t s) {
  if (R <= 0 || C <= 0) return hipSuccess;
  if (C % 16 || R % 32) return hipErrorInvalidValue;
  const long vecs = (long)C * (R / 8);
  const int blocks = (int)std::min<long>((vecs + 255) / 256, 8192);
  hipLaunchKernelGGL(k_frag_pack_t, dim3(blocks), dim3(256), 0, s, src, R, C, dst);
  return hipGetLastError();
}

hipError_t frag_pack(const uint16_t* src, int N, int K, uint16_t* dst, hipStream_t s) {
  if (N <= 0 || K <= 0) return hipSuccess;
  if (N % 16 || K % 32) return hipErrorInvalidValue;
  const long vecs = (long)N * (K / 8);
  const int blocks = (int)std::min<long>((vecs + 255) / 256, 8192);
  hipLaunchKernelGGL(k_frag_pack, dim3(blocks), dim3(256), 0, s, (const u32x4_t*)src, N, K, dst);
  return hipGetLastError();
}

// ------------------------------------------------------------------ fp32 SIMT
__global__ __launch_bounds__(256) void k_gemm_f32(const float* A, int lda, const float* W, int ldw, int M, int N,
                                                  int K, Epilogue e) {
  __shared__ float sA[16][64 + 4], sW[16][64 + 4];
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int el = threadIdx.x + i * 256, r = el >> 4, c = el & 15;
      sA[c][r] = (m0 + r < M) ? A[(long)(m0 + r) * lda + k0 + c] : 0.f;
      sW[c][r] = (n0 + r < N) ? W[(long)(n0 + r) * ldw + k0 + c] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = sA[kk][ty * 4 + i];
        w[i] = sW[kk][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], w[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (e.kind == EPI_GEGLU) {
        // columns 16 apart pair up: thread tx holds 4 columns, its partner is tx ^ 4
        const float other = __shfl_xor(acc[i][j], 4, 64);
        if (!(tx & 4) && m < M && n < N) epi_geglu(e, m, (n >> 5) * 16 + (n & 15), acc[i][j], other);
      } else if (m < M && n < N) {
        epi_store(e, m, n, acc[i][j]);
      }
    }
  }
}

hipError_t gemm_f32(const float* A, int lda, const float* W, int ldw, int M, int N, int K, const Epilogue& epi,
                    hipStream_t s) {
  if (M <= 0 || N <= 0 || K <= 0) return hipSuccess;
  if (K % 16 || (epi.kind == EPI_GEGLU && N % 32)) return hipErrorInvalidValue;
  dim3 grid((N + 63) / 64, (M + 63) / 64);
  hipLaunchKernelGGL(k_gemm_f32, grid, dim3(256), 0, s, A, lda, W, ldw, M, N, K, epi);
  return hipGetLastError();
}

}  // namespace vla
