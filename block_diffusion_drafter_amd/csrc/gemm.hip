// Weight-streaming GEMM for the drafter's projections: Y = A · W^T, A [M, K]
// (activations, M = rows of the draft block(s), small), W [N, K] row-major.
//
// At the block sizes of a drafting round (M = 16 per sequence) every
// projection is a stream of the weight matrix through HBM with 16 flops per
// byte, so the kernel is organised for bandwidth:
//   * a workgroup owns 16 output columns (one MFMA n-tile) and all M rows
//     (up to 4 m-tiles); its waves split K and meet in LDS at the end, so a
//     weight byte is read exactly once per launch;
//   * each lane streams 64 contiguous bytes of one weight row per chunk, four
//     lanes cover 256 contiguous bytes of the row; the next chunk is loaded
//     while the current one is multiplied;
//   * the k order inside a chunk is permuted identically for A and W (see
//     common.h), which the dot product does not see.
// Epilogues: fp32 store, fp32 residual add (x += acc), SwiGLU of a gate and an
// up stream computed side by side, and the LM head's per-row (max, argmax)
// over the tile (keys reduced across tiles by a second kernel).
#include "common.h"
#include "internal.h"

namespace dflash {

template <typename T> struct GemmGeom {
  static constexpr int EPF = 16 / (int)sizeof(T);   // elements per 16-byte fragment
  static constexpr int SPAN = 64 / (int)sizeof(T);  // contiguous k per lane per chunk
  static constexpr int KC = 4 * SPAN;               // k per chunk (4 lane groups)
};

template <typename T, int MT, int NB>
struct GemmRegs {
  u32x4 w[NB][4];
  u32x4 a[MT][4];
};

// Largest workgroup for a variant: wide variants (more m-tiles, two weight
// streams) need up to 256 VGPRs, i.e. at most 8 waves per workgroup.
template <int MT, int EPI>
constexpr int gemm_max_threads() {
  return (MT == 1 || (MT == 2 && EPI != EPI_SWIGLU)) ? 1024 : 512;
}

template <typename T, int MT, int EPI>
__global__ __launch_bounds__((gemm_max_threads<MT, EPI>())) void gemm_skinny_kernel(GemmArgs p) {
  constexpr int EPF = GemmGeom<T>::EPF;
  constexpr int SPAN = GemmGeom<T>::SPAN;
  constexpr int KC = GemmGeom<T>::KC;
  constexpr int NB = (EPI == EPI_SWIGLU) ? 2 : 1;
  extern __shared__ f32x4 red[];  // [ksplit][NB][MT][64]

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int ksplit = blockDim.x >> 6;
  const int r = lane & 15, grp = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int m_base = blockIdx.y * (16 * MT);
  const int n = n0 + r;
  const bool n_ok = n < p.N;

  const T* wrow[NB];
  {
    int s = 0;
    while (s + 1 < p.w_nseg && n >= p.w_row0[s + 1]) ++s;
    const int64_t row = n_ok ? (int64_t)(n - p.w_row0[s]) : 0;
    wrow[0] = reinterpret_cast<const T*>(p.w[s]) + row * p.K;
    if constexpr (NB == 2) wrow[1] = reinterpret_cast<const T*>(p.w2[s]) + row * p.K;
  }
  bool m_ok[MT];
  int64_t a_row_off[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = m_base + 16 * mt + r;
    m_ok[mt] = m < p.M;
    a_row_off[mt] = (int64_t)(m_ok[mt] ? m : 0) * p.a_stride;
  }

  const int k_begin = wave * p.k_per_wave;
  const int k_end = min(p.K, k_begin + p.k_per_wave);
  const int nchunks = k_end > k_begin ? (k_end - k_begin + KC - 1) / KC : 0;

  auto load = [&](GemmRegs<T, MT, NB>& g, int c) {
    const int kl = k_begin + c * KC + grp * SPAN;
    const int seg = kl / p.a_seg_k;  // SPAN divides a_seg_k: a lane never straddles segments
    const int koff = kl - seg * p.a_seg_k;
    const T* abase = reinterpret_cast<const T*>(p.a[seg < p.a_nseg ? seg : 0]) + koff;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const bool ok = kl + f * EPF < k_end;
#pragma unroll
      for (int b = 0; b < NB; ++b) g.w[b][f] = (ok && n_ok) ? ld16(wrow[b] + kl + f * EPF) : zero16();
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        g.a[mt][f] = (ok && m_ok[mt]) ? ld16(abase + a_row_off[mt] + f * EPF) : zero16();
    }
  };

  f32x4 acc[NB][MT];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[b][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const GemmRegs<T, MT, NB>& g) {
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[b][mt] = mfma_frag<T>(g.a[mt][f], g.w[b][f], acc[b][mt]);
  };

  if (nchunks > 0) {
    GemmRegs<T, MT, NB> g0, g1;
    load(g0, 0);
    for (int c = 0; c < nchunks; c += 2) {
      if (c + 1 < nchunks) load(g1, c + 1);
      compute(g0);
      if (c + 1 < nchunks) {
        if (c + 2 < nchunks) load(g0, c + 2);
        compute(g1);
      }
    }
  }

#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) red[((wave * NB + b) * MT + mt) * 64 + lane] = acc[b][mt];
  __syncthreads();
  if (wave >= MT) return;

  const int mt = wave;
  f32x4 v[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    v[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int w = 0; w < ksplit; ++w) v[b] += red[((w * NB + b) * MT + mt) * 64 + lane];
  }
  const int m0 = m_base + 16 * mt + 4 * grp;

  if constexpr (EPI == EPI_STORE_F32) {
    float* out = reinterpret_cast<float*>(p.out);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (m0 + i < p.M && n_ok) out[(int64_t)(m0 + i) * p.out_stride + n] = v[0][i];
  } else if constexpr (EPI == EPI_RESID) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (m0 + i < p.M && n_ok) p.resid[(int64_t)(m0 + i) * p.out_stride + n] += v[0][i];
  } else if constexpr (EPI == EPI_SWIGLU) {
    T* out = reinterpret_cast<T*>(p.out);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (m0 + i < p.M && n_ok) {
        const float gt = v[0][i];
        const float silu = gt / (1.0f + __expf(-gt));
        out[(int64_t)(m0 + i) * p.out_stride + n] = from_f32<T>(silu * v[1][i]);
      }
    }
  } else {  // EPI_ARGMAX
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + i;
      if (p.logits && m < p.M && n_ok) p.logits[(int64_t)m * p.logits_stride + n] = v[0][i];
      unsigned long long key = n_ok ? argmax_key(v[0][i], (unsigned)n) : 0ull;
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        const unsigned long long other = __shfl_xor(key, o);
        key = other > key ? other : key;
      }
      if (r == 0 && m < p.M) p.amax[(int64_t)m * p.amax_stride + blockIdx.x] = key;
    }
  }
}

template <typename T, int EPI>
static hipError_t launch_mt(int mt, dim3 grid, dim3 block, size_t lds, const GemmArgs& a,
                            hipStream_t st) {
  switch (mt) {
    case 1: hipLaunchKernelGGL((gemm_skinny_kernel<T, 1, EPI>), grid, block, lds, st, a); break;
    case 2: hipLaunchKernelGGL((gemm_skinny_kernel<T, 2, EPI>), grid, block, lds, st, a); break;
    case 3: hipLaunchKernelGGL((gemm_skinny_kernel<T, 3, EPI>), grid, block, lds, st, a); break;
    default: hipLaunchKernelGGL((gemm_skinny_kernel<T, 4, EPI>), grid, block, lds, st, a); break;
  }
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_t(int epi, int mt, dim3 grid, dim3 block, size_t lds, const GemmArgs& a,
                           hipStream_t st) {
  switch (epi) {
    case EPI_STORE_F32: return launch_mt<T, EPI_STORE_F32>(mt, grid, block, lds, a, st);
    case EPI_RESID: return launch_mt<T, EPI_RESID>(mt, grid, block, lds, a, st);
    case EPI_SWIGLU: return launch_mt<T, EPI_SWIGLU>(mt, grid, block, lds, a, st);
    default: return launch_mt<T, EPI_ARGMAX>(mt, grid, block, lds, a, st);
  }
}

hipError_t launch_gemm(int dtype, int epi, const GemmArgs& a0, hipStream_t st) {
  if (a0.M <= 0 || a0.N <= 0 || a0.K <= 0) return hipSuccess;
  GemmArgs a = a0;
  const int es = dtype == DFLASH_BF16 ? 2 : 4;
  const int KC = 4 * (64 / es);
  const int nb = epi == EPI_SWIGLU ? 2 : 1;
  const int mt = a.M >= 64 ? 4 : (a.M + 15) / 16;
  dim3 grid((a.N + 15) / 16, (a.M + 16 * mt - 1) / (16 * mt));
  const int chunks = (a.K + KC - 1) / KC;
  // Enough waves in flight to cover HBM latency, at least two chunks per wave.
  const int max_split = (mt == 1 || (mt == 2 && epi != EPI_SWIGLU)) ? 16 : 8;
  int ksplit = 4;
  const long long tiles = (long long)grid.x * grid.y;
  while (ksplit < max_split && tiles * ksplit < 8192 && chunks >= 4 * ksplit) ksplit *= 2;
  while (ksplit > 4 && (size_t)ksplit * nb * mt * 1024 > 65536) ksplit /= 2;
  a.k_per_wave = ((chunks + ksplit - 1) / ksplit) * KC;
  const size_t lds = (size_t)ksplit * nb * mt * 64 * sizeof(f32x4);
  dim3 block(64 * ksplit);
  if (dtype == DFLASH_BF16) return launch_t<bf16>(epi, mt, grid, block, lds, a, st);
  return launch_t<float>(epi, mt, grid, block, lds, a, st);
}

}  // namespace dflash
