// Weight-streaming GEMM for the drafter's projections: Y = A · W^T, A [M, K]
// (activations: the rows of the draft blocks, a few tens), W [N, K] row-major.
//
// At drafting sizes every projection is a stream of the weight matrix through
// HBM with ~16 flops per byte, so the kernel is organised for bandwidth:
//   * a workgroup owns NT·16 output columns and up to 64 rows; its waves split
//     K and meet in LDS at the end, so every weight byte is read once;
//   * per 256-byte chunk of a weight row, instruction f of lane (r, g) reads
//     bytes [64f + 16g, +16): one load instruction covers 64 contiguous bytes
//     of 16 rows, and the four instructions of a chunk cover 256 contiguous
//     bytes per row. That is the MFMA operand order itself (lane group g holds
//     k = 8g..8g+7 of each 32-wide step), so no data is shuffled;
//   * each wave carries NT n-tiles, so one activation fragment feeds NT MFMAs
//     and activation traffic (L2 hits) stays a fraction of the weight stream;
//   * chunk c+1 is in flight while chunk c is multiplied; interior tiles skip
//     all bounds predication.
// Epilogues: fp32 store, fp32 residual add (x += acc), SwiGLU of a gate and an
// up stream computed side by side, and the LM head's per-row (max, argmax)
// over each n-tile (keys reduced across tiles by a second kernel).
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace dflash {

template <typename T> struct GemmGeom {
  static constexpr int EPF = 16 / (int)sizeof(T);  // elements per 16-byte fragment
  static constexpr int KC = 16 * EPF;              // k per chunk: 4 fragments x 4 lane groups
};

template <int MT, int NT, int NB>
struct GemmRegs {
  u32x4 w[NB][NT][4];
  u32x4 a[MT][4];
};

// Chunks a wave loads per batch: 4 when four register buffers fit in ~160
// VGPRs (each holds (streams x n-tiles + m-tiles) x 16 registers), else 2.
constexpr int gemm_stages(int mt, int nt_streams) {
  return 4 * (nt_streams + mt) * 16 <= 160 ? 4 : 2;
}

// Registers of a variant allow 4 waves/SIMD (1024-thread groups) when the
// fragments in flight are few, else 2 waves/SIMD (512).
constexpr int gemm_threads_for(int mt, int nt_streams) {
  return gemm_stages(mt, nt_streams) * (mt + nt_streams) * 16 + 4 * mt * nt_streams <= 100 ? 1024
                                                                                         : 512;
}

template <typename T, int MT, int NT, int EPI>
__global__ __launch_bounds__((gemm_threads_for(MT, NT * (EPI == EPI_SWIGLU ? 2 : 1))))
void gemm_stream_kernel(GemmArgs p) {
  constexpr int EPF = GemmGeom<T>::EPF;
  constexpr int KC = GemmGeom<T>::KC;
  constexpr int NB = (EPI == EPI_SWIGLU) ? 2 : 1;
  constexpr int P = gemm_stages(MT, NB * NT);
  extern __shared__ f32x4 red[];  // [ksplit][NB][MT*NT][64]
  __shared__ unsigned long long kred[EPI == EPI_ARGMAX ? MT * 16 * NT : 1];

  const int lane = threadIdx.x & 63;
  // Wave-uniform values live in scalar registers: chunk and segment indices
  // derived from them never need vector loads (or their waits) in the loop.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ksplit = blockDim.x >> 6;
  const int r = lane & 15, grp = lane >> 4;
  const int n0 = blockIdx.x * (16 * NT);
  const int m_base = blockIdx.y * (16 * MT);
  const bool tile_full = n0 + 16 * NT <= p.N;

  // Weight row pointers: the lane's row in each n-tile, offset by its lane group.
  const T* wrow[NB][NT];
  bool n_ok[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int n = n0 + 16 * t + r;
    n_ok[t] = n < p.N;
    const int nn = n_ok[t] ? n : n0;
    int s = 0;
    while (s + 1 < p.w_nseg && nn >= p.w_row0[s + 1]) ++s;
    const int64_t row = nn - p.w_row0[s];
    wrow[0][t] = reinterpret_cast<const T*>(p.w[s]) + row * p.K + grp * EPF;
    if constexpr (NB == 2)
      wrow[1][t] = reinterpret_cast<const T*>(p.w2[s]) + row * p.K + grp * EPF;
  }
  // Rows past M read row M-1 (valid memory); their results are never stored.
  bool m_ok[MT];
  int64_t a_row_off[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = m_base + 16 * mt + r;
    m_ok[mt] = m < p.M;
    a_row_off[mt] = (int64_t)(m_ok[mt] ? m : p.M - 1) * p.a_stride + grp * EPF;
  }

  const int k_begin = wave * p.k_per_wave;
  const int k_end = min(p.K, k_begin + p.k_per_wave);
  const int nchunks = k_end > k_begin ? (k_end - k_begin + KC - 1) / KC : 0;
  // Chunks that need no bounds checks at all.
  const int n_full = tile_full ? max(0, (k_end - k_begin) / KC) : 0;
  // A operand: a wave's K range never crosses an A segment (the host sizes
  // the split so), so the segment is resolved once, before the loop, and the
  // loop addresses A linearly from this wave's base.
  const int seg0 = __builtin_amdgcn_readfirstlane(k_begin / p.a_seg_k);
  const T* a_wave = reinterpret_cast<const T*>(p.a[seg0 < p.a_nseg ? seg0 : 0]) +
                    (k_begin - seg0 * p.a_seg_k) - k_begin;
  auto a_base = [&](int kc) -> const T* { return a_wave + kc; };

  auto load_full = [&](GemmRegs<MT, NT, NB>& g, int c) {
    const int kc = k_begin + c * KC;
    const T* ab = a_base(kc);
#pragma unroll
    for (int f = 0; f < 4; ++f) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int t = 0; t < NT; ++t) g.w[b][t][f] = ld16(wrow[b][t] + kc + f * 4 * EPF);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) g.a[mt][f] = ld16(ab + a_row_off[mt] + f * 4 * EPF);
    }
  };

  auto load_checked = [&](GemmRegs<MT, NT, NB>& g, int c) {
    const int kc = k_begin + c * KC;
    const T* ab = a_base(kc);
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const bool ok = kc + f * 4 * EPF + grp * EPF < k_end;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int t = 0; t < NT; ++t)
          g.w[b][t][f] = (ok && n_ok[t]) ? ld16(wrow[b][t] + kc + f * 4 * EPF) : zero16();
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        g.a[mt][f] = ok ? ld16(ab + a_row_off[mt] + f * 4 * EPF) : zero16();
    }
  };

  f32x4 acc[NB][MT][NT];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[b][mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const GemmRegs<MT, NT, NB>& g) {
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int t = 0; t < NT; ++t)
            acc[b][mt][t] = mfma_frag<T>(g.a[mt][f], g.w[b][t][f], acc[b][mt][t]);
  };

  // Main loop: batches of P full chunks. Each batch issues all of its loads,
  // then multiplies them; nothing is carried from one batch to the next, so
  // the compiler's wait counts inside a batch are exact (partial), and the
  // other waves on the SIMD cover the gap between batches. The host sizes
  // each wave's K range as a multiple of P chunks where it can.
  const int n_batched = (n_full / P) * P;
  for (int base = 0; base < n_batched; base += P) {
    GemmRegs<MT, NT, NB> buf[P];
#pragma unroll
    for (int s = 0; s < P; ++s) load_full(buf[s], base + s);
    // Keep every load of the batch ahead of its first MFMA.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < P; ++s) compute(buf[s]);
    __builtin_amdgcn_sched_barrier(0);
  }
  // Tail: leftover chunks, the partial chunk at the end of K, or every chunk
  // of the last column tile when it is ragged.
  for (int c = n_batched; c < nchunks; ++c) {
    GemmRegs<MT, NT, NB> g;
    load_checked(g, c);
    compute(g);
  }

  constexpr int PAIRS = MT * NT;
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int t = 0; t < NT; ++t)
        red[((wave * NB + b) * PAIRS + mt * NT + t) * 64 + lane] = acc[b][mt][t];
  __syncthreads();

  // Wave w finishes output tiles w, w + ksplit, ... of the MT x NT grid.
  for (int pi = wave; pi < PAIRS; pi += ksplit) {
    const int mt = pi / NT, t = pi % NT;
    f32x4 v[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      v[b] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int w = 0; w < ksplit; ++w) v[b] += red[((w * NB + b) * PAIRS + pi) * 64 + lane];
    }
    const int m0 = m_base + 16 * mt + 4 * grp;
    const int n = n0 + 16 * t + r;
    const bool nok = n < p.N;
    if constexpr (EPI == EPI_STORE_F32) {
      float* out = reinterpret_cast<float*>(p.out);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (m0 + i < p.M && nok) out[(int64_t)(m0 + i) * p.out_stride + n] = v[0][i];
    } else if constexpr (EPI == EPI_RESID) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (m0 + i < p.M && nok) p.resid[(int64_t)(m0 + i) * p.out_stride + n] += v[0][i];
    } else if constexpr (EPI == EPI_SWIGLU) {
      T* out = reinterpret_cast<T*>(p.out);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (m0 + i < p.M && nok) {
          const float gt = v[0][i];
          const float silu = gt / (1.0f + __expf(-gt));
          out[(int64_t)(m0 + i) * p.out_stride + n] = from_f32<T>(silu * v[1][i]);
        }
      }
    } else {  // EPI_ARGMAX: one (max, argmax) key per row and n-tile, merged below
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + i;
        if (p.logits && m < p.M && nok) p.logits[(int64_t)m * p.logits_stride + n] = v[0][i];
        unsigned long long key = nok ? argmax_key(v[0][i], (unsigned)n) : 0ull;
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
          const unsigned long long other = __shfl_xor(key, o);
          key = other > key ? other : key;
        }
        if (r == 0) kred[(16 * mt + 4 * grp + i) * NT + t] = key;
      }
    }
  }
  if constexpr (EPI == EPI_ARGMAX) {
    __syncthreads();
    // One key per row for the whole workgroup (keys of empty tiles are 0).
    const int row = threadIdx.x;
    if (row < 16 * MT && m_base + row < p.M) {
      unsigned long long best = 0ull;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const unsigned long long k = kred[row * NT + t];
        best = k > best ? k : best;
      }
      p.amax[(int64_t)(m_base + row) * p.amax_stride + blockIdx.x] = best;
    }
  }
}

template <typename T, int MT, int NT, int EPI>
static void launch_one(dim3 grid, dim3 block, size_t lds, const GemmArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((gemm_stream_kernel<T, MT, NT, EPI>), grid, block, lds, st, a);
}

template <typename T, int EPI>
static hipError_t dispatch(int mt, int nt, dim3 grid, dim3 block, size_t lds, const GemmArgs& a,
                           hipStream_t st) {
  if constexpr (sizeof(T) == 4) {  // fp32 drafters: one n-tile per wave
    switch (mt) {
      case 1: launch_one<T, 1, 1, EPI>(grid, block, lds, a, st); break;
      case 2: launch_one<T, 2, 1, EPI>(grid, block, lds, a, st); break;
      case 3: launch_one<T, 3, 1, EPI>(grid, block, lds, a, st); break;
      default: launch_one<T, 4, 1, EPI>(grid, block, lds, a, st); break;
    }
  } else if constexpr (EPI == EPI_SWIGLU) {  // two weight streams: fewer n-tiles fit
    switch (mt * 10 + nt) {
      case 11: launch_one<T, 1, 1, EPI>(grid, block, lds, a, st); break;
      case 12: launch_one<T, 1, 2, EPI>(grid, block, lds, a, st); break;
      case 21: launch_one<T, 2, 1, EPI>(grid, block, lds, a, st); break;
      case 31: launch_one<T, 3, 1, EPI>(grid, block, lds, a, st); break;
      default: launch_one<T, 4, 1, EPI>(grid, block, lds, a, st); break;
    }
  } else {
    switch (mt * 10 + nt) {
      case 11: launch_one<T, 1, 1, EPI>(grid, block, lds, a, st); break;
      case 12: launch_one<T, 1, 2, EPI>(grid, block, lds, a, st); break;
      case 14: launch_one<T, 1, 4, EPI>(grid, block, lds, a, st); break;
      case 21: launch_one<T, 2, 1, EPI>(grid, block, lds, a, st); break;
      case 22: launch_one<T, 2, 2, EPI>(grid, block, lds, a, st); break;
      case 31: launch_one<T, 3, 1, EPI>(grid, block, lds, a, st); break;
      default: launch_one<T, 4, 1, EPI>(grid, block, lds, a, st); break;
    }
  }
  return hipGetLastError();
}

GemmPlan plan_gemm(int dtype, int epi, int M, int N, int K, int a_seg_k) {
  GemmPlan g{};
  const bool bf = dtype == DFLASH_BF16;
  const int KC = bf ? 128 : 64;
  const bool multi_seg = a_seg_k > 0 && a_seg_k < K;
  if (!multi_seg) a_seg_k = ((K + KC - 1) / KC) * KC;
  const int nb = epi == EPI_SWIGLU ? 2 : 1;
  g.mt = M >= 64 ? 4 : (M + 15) / 16;
  const int chunks = (K + KC - 1) / KC;
  const int col_tiles = (N + 15) / 16;
  // Widest n-tiling (fewer activation re-reads) that still leaves >= 1024
  // workgroups, i.e. several per CU on all 256 CUs.
  g.nt = 1;
  if (bf) {
    // Register budget (256 VGPRs at 2 waves/SIMD) bounds the double-buffered
    // fragments: (streams x n-tiles + m-tiles) <= 5 chunks of 16 registers.
    const int max_nt = g.mt == 1 ? (nb == 2 ? 2 : 4) : (g.mt == 2 && nb == 1 ? 2 : 1);
    const long long rows_wg = (M + 16 * g.mt - 1) / (16 * g.mt);
    while (g.nt < max_nt && (long long)((col_tiles + 2 * g.nt - 1) / (2 * g.nt)) * rows_wg >= 1024)
      g.nt *= 2;
  }
  g.grid_x = (N + 16 * g.nt - 1) / (16 * g.nt);
  g.grid_y = (M + 16 * g.mt - 1) / (16 * g.mt);
  const int max_split = gemm_threads_for(g.mt, g.nt * nb) / 64;
  const int stages = gemm_stages(g.mt, g.nt * nb);
  const long long tiles = (long long)g.grid_x * g.grid_y;
  // Waves per workgroup (K split): prefer splits that give every wave a whole
  // number of P-chunk batches, then enough waves in flight (>= 8192 over the
  // grid) to cover HBM latency, then longer runs per wave. With several A
  // segments (fused features), a wave's range must stay inside one segment.
  const int seg_chunks = a_seg_k / KC;
  g.ksplit = 0;
  long long best = -1;
  for (int ks = 1; ks <= max_split; ++ks) {
    if ((size_t)ks * nb * g.mt * g.nt * 1024 > 65536) break;
    const int per = (chunks + ks - 1) / ks;
    if (multi_seg && seg_chunks % per) continue;
    if (!multi_seg && ks < 4 && chunks >= 4) continue;
    const bool exact = chunks % (ks * stages) == 0 && chunks / ks >= stages;
    const long long waves = tiles * ks;
    const long long score = (exact ? 4LL : 0LL) * 1000000 + std::min(waves, 8192LL) * 100 +
                            std::min(per, 16);
    if (score > best) {
      best = score;
      g.ksplit = ks;
    }
  }
  if (g.ksplit == 0) return g;  // no valid split: the caller reports the shape as unsupported
  g.k_per_wave = ((chunks + g.ksplit - 1) / g.ksplit) * KC;
  g.lds = (size_t)g.ksplit * nb * g.mt * g.nt * 64 * sizeof(f32x4);
  return g;
}

hipError_t launch_gemm(int dtype, int epi, const GemmArgs& a0, hipStream_t st) {
  if (a0.M <= 0 || a0.N <= 0 || a0.K <= 0) return hipSuccess;
  const GemmPlan g = plan_gemm(dtype, epi, a0.M, a0.N, a0.K, a0.a_nseg > 1 ? a0.a_seg_k : 0);
  if (g.ksplit == 0) return hipErrorInvalidValue;
  GemmArgs a = a0;
  a.k_per_wave = g.k_per_wave;
  dim3 grid(g.grid_x, g.grid_y), block(64 * g.ksplit);
  if (dtype == DFLASH_BF16) {
    switch (epi) {
      case EPI_STORE_F32: return dispatch<bf16, EPI_STORE_F32>(g.mt, g.nt, grid, block, g.lds, a, st);
      case EPI_RESID: return dispatch<bf16, EPI_RESID>(g.mt, g.nt, grid, block, g.lds, a, st);
      case EPI_SWIGLU: return dispatch<bf16, EPI_SWIGLU>(g.mt, g.nt, grid, block, g.lds, a, st);
      default: return dispatch<bf16, EPI_ARGMAX>(g.mt, g.nt, grid, block, g.lds, a, st);
    }
  }
  switch (epi) {
    case EPI_STORE_F32: return dispatch<float, EPI_STORE_F32>(g.mt, 1, grid, block, g.lds, a, st);
    case EPI_RESID: return dispatch<float, EPI_RESID>(g.mt, 1, grid, block, g.lds, a, st);
    case EPI_SWIGLU: return dispatch<float, EPI_SWIGLU>(g.mt, 1, grid, block, g.lds, a, st);
    default: return dispatch<float, EPI_ARGMAX>(g.mt, 1, grid, block, g.lds, a, st);
  }
}

}  // namespace dflash
