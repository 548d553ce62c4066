// Weight-streaming GEMM for the drafter's projections: Y = A · W^T, A [M, K]
// (activations: the rows of the draft blocks, a few tens), W [N, K].
//
// At drafting sizes every projection is a stream of the weight matrix through
// HBM with ~16 flops per byte, so the kernel is organised for bandwidth:
//   * a workgroup owns NT·16 output columns and up to 64 rows; its waves split
//     K and meet in LDS at the end, so every weight byte is read once;
//   * weights (always) and workspace activations are in the tiled layout of
//     common.h: each load instruction of a wave reads one contiguous 1 KB
//     fragment, which is the MFMA operand itself, so nothing is shuffled and
//     the memory system sees whole lines. (With row-major operands a wave's
//     load touches 16 rows x 64 bytes; the activation loads then cost as much
//     as the weight stream although they hit in L2.)
//   * each wave carries NT n-tiles, so one activation fragment feeds NT MFMAs;
//   * loads go out in batches of P chunks before the batch's MFMAs; weight
//     loads never need bounds checks (padded tiles, clamped tile indices).
// Caller-provided row-major activations (the target features, context rows)
// are read through the row-major path.
// Epilogues: fp32 store, fp32 residual add (x += acc), SwiGLU of a gate and an
// up stream computed side by side (tiled output: the next GEMM's A), and the
// LM head's per-row (max, argmax) over each n-tile (keys reduced across tiles
// by a second kernel).
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

template <typename T, int MT, int NT, int EPI, bool AT>
__global__ __launch_bounds__((gemm_threads_for(MT, NT * (EPI == EPI_SWIGLU ? 2 : 1))))
void gemm_stream_kernel(GemmArgs p) {
  constexpr int EPF = GemmGeom<T>::EPF;
  constexpr int KC = GemmGeom<T>::KC;
  constexpr int FRAG = 64 * EPF;  // elements of one wave-wide 1 KB fragment
  constexpr int NB = (EPI == EPI_SWIGLU) ? 2 : 1;
  constexpr int P = gemm_stages(MT, NB * NT);
  extern __shared__ f32x4 red[];  // [ksplit][NB][MT*NT][64]
  __shared__ unsigned long long kred[EPI == EPI_ARGMAX ? MT * 16 * NT : 1];
  // Deferred RMSNorm of the A rows (sq_in): per-thread partial sums, then the
  // rows' scales.
  constexpr bool SQ = (EPI == EPI_STORE_F32 || EPI == EPI_SWIGLU) && MT == 1;
  constexpr int SQV = 2;  // float4 partials a thread holds: tiles <= 4 * SQV * threads / 16
  __shared__ float sq_part[SQ ? 1024 : 1];
  __shared__ float row_inv[SQ ? 16 * MT : 1];

  if constexpr (EPI == EPI_STORE_F32) gemm_snapshot(p, blockIdx.x == 0 && blockIdx.y == 0);
  const int lane = threadIdx.x & 63;
  // Wave-uniform values live in scalar registers: chunk indices derived from
  // them never need vector loads (or their waits) in the loop.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ksplit = blockDim.x >> 6;
  const int r = lane & 15, grp = lane >> 4;
  const int nck = (p.K + KC - 1) / KC;
  const int n_tiles = (p.N + 15) >> 4;
  const int tile0 = blockIdx.x * NT;
  const int m_base = blockIdx.y * (16 * MT);

  // Deferred norm (one m-tile): thread t loads the tile partials 4 j .. 4 j + 3,
  // j = t / 16 + u * nparts (u < SQV), of row t % 16 now, ahead of the weight
  // stream, and adds them after the main loop (so no wait on them before it).
  float4 sqv[SQ ? SQV : 1];
  if constexpr (SQ) {
    const int nparts = (int)blockDim.x / 16, part = threadIdx.x / 16;
    const int m = m_base + (int)(threadIdx.x % 16), tiles4 = (((p.sq_d + 15) >> 4) + 3) >> 2;
#pragma unroll
    for (int u = 0; u < SQV; ++u) {
      const int j = part + u * nparts;
      sqv[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (p.sq_in && m < p.M && j < tiles4)
        sqv[u] = *reinterpret_cast<const float4*>(p.sq_in + ((int64_t)m * tiles4 + j) * 4);
    }
  }

  // Weight fragments of the lane in each n-tile. Tiles past the last one
  // re-read the last tile (valid memory); their columns are never stored.
  const T* wt[NB][NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int64_t off = (int64_t)min(tile0 + t, n_tiles - 1) * nck * 4 * FRAG + lane * EPF;
    wt[0][t] = reinterpret_cast<const T*>(p.w) + off;
    if constexpr (NB == 2) wt[1][t] = reinterpret_cast<const T*>(p.w2) + off;
  }

  const int k_begin = wave * p.k_per_wave;
  const int k_end = min(p.K, k_begin + p.k_per_wave);
  const int c_begin = k_begin / KC;
  const int nchunks = k_end > k_begin ? (k_end - k_begin + KC - 1) / KC : 0;
  // Chunks whose every k is inside K.
  const int n_full = max(0, (k_end - k_begin) / KC);

  // A operand. Tiled: per m-tile fragment base (tiles past the last re-read
  // it). Row-major: rows past M read row M-1; a wave's K range never crosses
  // an A segment (the host sizes the split so), so the segment is resolved
  // once and the loop addresses A linearly from this wave's base.
  int64_t a_off[MT];
  const T* a_wave;
  if constexpr (AT) {
    const int m_tiles = (p.M + 15) >> 4;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      a_off[mt] = (int64_t)min((int)blockIdx.y * MT + mt, m_tiles - 1) * nck * 4 * FRAG + lane * EPF;
    a_wave = reinterpret_cast<const T*>(p.a[0]);
  } else {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = m_base + 16 * mt + r;
      a_off[mt] = (int64_t)(m < p.M ? m : p.M - 1) * p.a_stride + grp * EPF;
    }
    const int seg0 = __builtin_amdgcn_readfirstlane(k_begin / p.a_seg_k);
    a_wave = reinterpret_cast<const T*>(p.a[seg0 < p.a_nseg ? seg0 : 0]) +
             (k_begin - seg0 * p.a_seg_k) - k_begin;
  }

  // Fragment f of chunk c (counted from this wave's first chunk).
  auto a_frag = [&](int mt, int c, int f) -> const T* {
    if constexpr (AT) return a_wave + a_off[mt] + (int64_t)((c_begin + c) * 4 + f) * FRAG;
    else return a_wave + a_off[mt] + k_begin + c * KC + f * 4 * EPF;
  };

  auto load_full = [&](GemmRegs<MT, NT, NB>& g, int c) {
#pragma unroll
    for (int f = 0; f < 4; ++f) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int t = 0; t < NT; ++t)
          g.w[b][t][f] = ld16(wt[b][t] + (int64_t)((c_begin + c) * 4 + f) * FRAG);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) g.a[mt][f] = ld16(a_frag(mt, c, f));
    }
  };

  // The chunk that crosses K: weights are zero-padded there, activations past
  // K are replaced by zeros (their memory is padding or another row).
  auto load_tail = [&](GemmRegs<MT, NT, NB>& g, int c) {
    const int kc = k_begin + c * KC;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const bool ok = kc + f * 4 * EPF + grp * EPF < k_end;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int t = 0; t < NT; ++t)
          g.w[b][t][f] = ld16(wt[b][t] + (int64_t)((c_begin + c) * 4 + f) * FRAG);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) g.a[mt][f] = ok ? ld16(a_frag(mt, c, f)) : zero16();
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
  // other waves on the SIMD cover the gap between batches (a wave that keeps
  // two batches in registers instead measured slower: half the batch, and
  // the SIMD's other waves already overlap). The host sizes each wave's K
  // range as a multiple of P chunks where it can.
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
  // Leftover full chunks, then the chunk that crosses K.
  for (int c = n_batched; c < n_full; ++c) {
    GemmRegs<MT, NT, NB> g;
    load_full(g, c);
    compute(g);
  }
  if (n_full < nchunks) {
    GemmRegs<MT, NT, NB> g;
    load_tail(g, n_full);
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
  if constexpr (SQ) {
    if (p.sq_in) {
      const int nparts = (int)blockDim.x / 16, part = threadIdx.x / 16;
      const int tiles = (p.sq_d + 15) >> 4;
      float sq_acc = 0.f;
#pragma unroll
      for (int u = 0; u < SQV; ++u) {
        const int j = 4 * (part + u * nparts);
        sq_acc += (j < tiles ? sqv[u].x : 0.f) + (j + 1 < tiles ? sqv[u].y : 0.f) +
                  (j + 2 < tiles ? sqv[u].z : 0.f) + (j + 3 < tiles ? sqv[u].w : 0.f);
      }
      // Partials beyond what the registers held (few threads, wide rows).
      const int m = m_base + (int)(threadIdx.x % 16), tiles4 = (tiles + 3) >> 2;
      for (int j4 = part + SQV * nparts; m < p.M && j4 < tiles4; j4 += nparts) {
        const float4 q = *reinterpret_cast<const float4*>(p.sq_in + ((int64_t)m * tiles4 + j4) * 4);
        const int j = 4 * j4;
        sq_acc += q.x + (j + 1 < tiles ? q.y : 0.f) + (j + 2 < tiles ? q.z : 0.f) +
                  (j + 3 < tiles ? q.w : 0.f);
      }
      sq_part[threadIdx.x] = sq_acc;
    }
  }
  __syncthreads();
  if constexpr (SQ) {
    if (p.sq_in) {
      const int rows_wg = 16 * MT, nparts = (int)blockDim.x / rows_wg;
      if ((int)threadIdx.x < rows_wg) {
        float ss = 0.f;
        for (int k = 0; k < nparts; ++k) ss += sq_part[k * rows_wg + threadIdx.x];
        row_inv[threadIdx.x] = rsqrtf(ss / (float)p.sq_d + p.norm_eps);
      }
      __syncthreads();
    }
  }

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
    const int n = 16 * (tile0 + t) + r;
    const bool nok = n < p.N;
    if constexpr (SQ) {
      if (p.sq_in) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float s = row_inv[16 * mt + 4 * grp + i];
#pragma unroll
          for (int b = 0; b < NB; ++b) v[b][i] *= s;
        }
      }
    }
    if constexpr (EPI == EPI_STORE_F32) {
      float* out = reinterpret_cast<float*>(p.out);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (m0 + i < p.M && nok) out[(int64_t)(m0 + i) * p.out_stride + n] = v[0][i];
    } else if constexpr (EPI == EPI_RESID) {
      float xn[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xn[i] = 0.f;
        if (m0 + i < p.M && nok) {
          float* px = p.resid + (int64_t)(m0 + i) * p.out_stride + n;
          xn[i] = *px + v[0][i];
          *px = xn[i];
        }
      }
      if (p.sq_out) {
        // The next norm's input, bf16(x * gain) tiled, and each row's sum of
        // squares over this tile's 16 columns (lanes r = 0..15 of a group).
        const float gain = nok ? to_f32(reinterpret_cast<const T*>(p.norm_w)[n]) : 0.f;
        T* hn = reinterpret_cast<T*>(p.norm_out);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (m0 + i < p.M && nok) hn[tiled_index<T>(m0 + i, n, p.norm_nck)] = from_f32<T>(xn[i] * gain);
          float sq = xn[i] * xn[i];
#pragma unroll
          for (int o = 1; o < 16; o <<= 1) sq += __shfl_xor(sq, o);
          if (r == 0 && m0 + i < p.M && tile0 + t < n_tiles)
            p.sq_out[(int64_t)(m0 + i) * ((n_tiles + 3) & ~3) + tile0 + t] = sq;
        }
      }
    } else if constexpr (EPI == EPI_SWIGLU) {
      // Tiled output [M, N]: the A operand of the down projection.
      T* out = reinterpret_cast<T*>(p.out);
      const int out_nck = (p.N + KC - 1) / KC;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (m0 + i < p.M && nok) {
          const float gt = v[0][i];
          const float silu = gt / (1.0f + __expf(-gt));
          out[tiled_index<T>(m0 + i, n, out_nck)] = from_f32<T>(silu * v[1][i]);
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

template <typename T, int MT, int NT, int EPI, bool AT>
static void launch_one(dim3 grid, dim3 block, size_t lds, const GemmArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((gemm_stream_kernel<T, MT, NT, EPI, AT>), grid, block, lds, st, a);
}

// The (MT, NT) pairs plan_gemm produces; anything else is refused.
template <typename T, int EPI, bool AT>
static hipError_t dispatch(int mt, int nt, dim3 grid, dim3 block, size_t lds, const GemmArgs& a,
                           hipStream_t st) {
  switch (mt * 10 + nt) {
    case 11: launch_one<T, 1, 1, EPI, AT>(grid, block, lds, a, st); break;
    case 21: launch_one<T, 2, 1, EPI, AT>(grid, block, lds, a, st); break;
    case 31: launch_one<T, 3, 1, EPI, AT>(grid, block, lds, a, st); break;
    case 41: launch_one<T, 4, 1, EPI, AT>(grid, block, lds, a, st); break;
    case 22:
      if constexpr (sizeof(T) == 2 && EPI != EPI_SWIGLU) {
        launch_one<T, 2, 2, EPI, AT>(grid, block, lds, a, st);
        break;
      }
      return hipErrorInvalidValue;
    case 32:
      if constexpr (sizeof(T) == 2 && EPI != EPI_SWIGLU) {
        launch_one<T, 3, 2, EPI, AT>(grid, block, lds, a, st);
        break;
      }
      return hipErrorInvalidValue;
    case 42:
      if constexpr (sizeof(T) == 2 && EPI != EPI_SWIGLU) {
        launch_one<T, 4, 2, EPI, AT>(grid, block, lds, a, st);
        break;
      }
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
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
  // n-tiles per wave. With one m-tile, activation fragments are a small
  // share of the traffic once they are tiled, and one n-tile per wave keeps
  // the deepest load batches: it measured best or equal at every drafting
  // shape (LM head, QKV, O, gate/up, down). With several m-tiles each weight
  // fragment already feeds MT MFMAs, and every workgroup re-reads all of its
  // rows' activations from L2; two n-tiles halve those re-reads where
  // registers allow: always from three m-tiles (LM head at 60 rows: 379 ->
  // 269 us; 60-row projections -10 to -26%), at two as long as >= 1024
  // workgroups remain.
  g.nt = 1;
  if (bf && g.mt >= 3 && nb == 1) {
    g.nt = 2;
  } else if (bf && g.mt == 2 && nb == 1) {
    const long long rows_wg = (M + 16 * g.mt - 1) / (16 * g.mt);
    if ((long long)((col_tiles + 1) / 2) * rows_wg >= 1024) g.nt = 2;
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

int gemm_amax_cols(int dtype, int M, int N, int K) {
  if (gemm_uses_mfma(dtype, M, K, true, EPI_ARGMAX)) return mfma_argmax_keys(M, N, K);
  return plan_gemm(dtype, EPI_ARGMAX, M, N, K, 0).grid_x;
}

hipError_t launch_gemm(int dtype, int epi, const GemmArgs& a0, hipStream_t st) {
  if (a0.M <= 0 || a0.N <= 0 || a0.K <= 0) return hipSuccess;
  if (gemm_uses_mfma(dtype, a0.M, a0.K, a0.a_tiled != 0, epi)) return launch_gemm_mfma(epi, a0, st);
  // Row-major activations only come from callers, as inputs of fp32-output projections.
  if (!a0.a_tiled && epi != EPI_STORE_F32) return hipErrorInvalidValue;
  const bool multi = !a0.a_tiled && a0.a_nseg > 1;
  const GemmPlan g = plan_gemm(dtype, epi, a0.M, a0.N, a0.K, multi ? a0.a_seg_k : 0);
  if (g.ksplit == 0) return hipErrorInvalidValue;
  GemmArgs a = a0;
  a.k_per_wave = g.k_per_wave;
  if (!multi) a.a_seg_k = g.k_per_wave * g.ksplit;  // one segment covering every wave's range
  dim3 grid(g.grid_x, g.grid_y), block(64 * g.ksplit);
  if (dtype == DFLASH_BF16) {
    if (!a.a_tiled) return dispatch<bf16, EPI_STORE_F32, false>(g.mt, g.nt, grid, block, g.lds, a, st);
    switch (epi) {
      case EPI_STORE_F32: return dispatch<bf16, EPI_STORE_F32, true>(g.mt, g.nt, grid, block, g.lds, a, st);
      case EPI_RESID: return dispatch<bf16, EPI_RESID, true>(g.mt, g.nt, grid, block, g.lds, a, st);
      case EPI_SWIGLU: return dispatch<bf16, EPI_SWIGLU, true>(g.mt, g.nt, grid, block, g.lds, a, st);
      default: return dispatch<bf16, EPI_ARGMAX, true>(g.mt, g.nt, grid, block, g.lds, a, st);
    }
  }
  if (!a.a_tiled) return dispatch<float, EPI_STORE_F32, false>(g.mt, 1, grid, block, g.lds, a, st);
  switch (epi) {
    case EPI_STORE_F32: return dispatch<float, EPI_STORE_F32, true>(g.mt, 1, grid, block, g.lds, a, st);
    case EPI_RESID: return dispatch<float, EPI_RESID, true>(g.mt, 1, grid, block, g.lds, a, st);
    case EPI_SWIGLU: return dispatch<float, EPI_SWIGLU, true>(g.mt, 1, grid, block, g.lds, a, st);
    default: return dispatch<float, EPI_ARGMAX, true>(g.mt, 1, grid, block, g.lds, a, st);
  }
}

// One thread per 16-byte fragment of the tiled destination.
template <typename T>
__global__ __launch_bounds__(256) void pack_tiled_kernel(PackSrc src, int rows, int K, int nck,
                                                         int64_t n_frags, T* __restrict__ dst) {
  constexpr int EPF = GemmGeom<T>::EPF;
  constexpr int KC = GemmGeom<T>::KC;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_frags; i += stride) {
    const int lane = (int)(i & 63);
    const int64_t q = i >> 6;
    const int f = (int)(q & 3);
    const int64_t blk = q >> 2;
    const int c = (int)(blk % nck);
    const int64_t tile = blk / nck;
    const int64_t row = tile * 16 + (lane & 15);
    const int k = c * KC + f * 4 * EPF + (lane >> 4) * EPF;
    u32x4 v = zero16();
    if (row < rows && k < K) {
      const int sg = k / src.seg_k;
      const T* base = reinterpret_cast<const T*>(src.seg[sg]);
      v = ld16(base + row * src.row_stride + (k - sg * src.seg_k));
    }
    *reinterpret_cast<u32x4*>(dst + i * EPF) = v;
  }
}

hipError_t launch_pack_tiled(int dtype, const PackSrc& src, int rows, int K, void* dst,
                             hipStream_t st) {
  if (rows <= 0 || K <= 0) return hipSuccess;
  const int epf = dtype == DFLASH_BF16 ? 8 : 4;
  // Whole 16-byte source fragments that never straddle a segment.
  if (src.seg_k % epf || src.row_stride % epf || src.nseg < 1 || src.nseg > kMaxASeg ||
      (int64_t)src.nseg * src.seg_k < K)
    return hipErrorInvalidValue;
  const int64_t n_frags = (int64_t)tiled_bytes(dtype, rows, K) / 16;
  const int64_t blocks = std::min<int64_t>((n_frags + 255) / 256, 8192);
  const int nck = tiled_nck(dtype, K);
  if (dtype == DFLASH_BF16)
    hipLaunchKernelGGL(pack_tiled_kernel<bf16>, dim3((unsigned)blocks), dim3(256), 0, st, src,
                       rows, K, nck, n_frags, (bf16*)dst);
  else
    hipLaunchKernelGGL(pack_tiled_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, st, src,
                       rows, K, nck, n_frags, (float*)dst);
  return hipGetLastError();
}

}  // namespace dflash
