// KV-injected attention of the draft block over [cached context ; block] keys.
//
// The block's queries (B <= 16 rows per head) attend non-causally to every
// cached context position of their sequence plus the block's own keys, which
// the QKV step has already staged in the cache's scratch positions
// [ctx_len, ctx_len + B). With 16 queries per head over thousands of keys the
// work is a stream of the K/V cache, split over key chunks:
//
//   attn_partial: one workgroup per (sequence, KV head, key chunk), one wave
//     per query head of the GQA group. The waves of a group read the same K/V
//     positions, so after the first wave the loads hit the CU's L1: HBM sees
//     each position once. Scores are computed transposed, S^T = K Q^T (keys as
//     MFMA rows, queries as columns), and the output likewise, O^T = V^T P^T,
//     so each lane owns one query column: the online-softmax running max/sum
//     are per-lane values plus a two-step shuffle across the four lane groups.
//     P leaves the S^T accumulator already in the layout the next MFMA's B
//     operand needs (the key order inside a 32-key block is permuted to make
//     that so). V is stored channel-major inside 32-position blocks, so each
//     lane's V fragment is one 16-byte load. The next block's K/V is loaded
//     while the current one is multiplied. A sequence that fits in one chunk
//     is normalised and written directly; otherwise the chunk's (max, sum,
//     unnormalised O) go to a partial buffer.
//   attn_combine: merges the chunks of the sequences that needed several.
#include "common.h"
#include "internal.h"

namespace dflash {

// Row r (0..15) of S^T tile t (0..1) of a 32-key block -> key offset in the block.
template <typename T>
__device__ __forceinline__ int key_of(int t, int r) {
  if constexpr (sizeof(T) == 2) {
    // bf16: the PV MFMA consumes 8 consecutive keys per lane group; lane group
    // g holds rows 4g..4g+3 of both tiles, so tile t row 4g+i is key 8g+4t+i.
    return 8 * (r >> 2) + 4 * t + (r & 3);
  } else {
    return 16 * t + r;  // fp32: one PV MFMA per 4 keys, natural order
  }
}

// Zero the elements of a 16-byte fragment whose index is >= nvalid.
template <typename T>
__device__ __forceinline__ u32x4 keep_first(u32x4 v, int nvalid) {
  constexpr int EPF = 16 / (int)sizeof(T);
  if (nvalid >= EPF) return v;
  if (nvalid <= 0) return zero16();
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int e0 = 2 * w;
      const unsigned mask = (e0 < nvalid ? 0x0000FFFFu : 0u) | (e0 + 1 < nvalid ? 0xFFFF0000u : 0u);
      v[w] &= mask;
    }
  } else {
#pragma unroll
    for (int w = 0; w < 4; ++w)
      if (w >= nvalid) v[w] = 0u;
  }
  return v;
}

__device__ __forceinline__ int seq_keys(const AttnArgs& p, int s) {
  int cl = p.ctx_len[s];
  cl = cl < 0 ? 0 : cl;
  return min(cl + p.block, p.cap);
}

template <typename T, int HD>
struct KVBlock {
  static constexpr int EPF = 16 / (int)sizeof(T);
  static constexpr int FR = (HD / 4) / EPF;           // K fragments per lane per key row
  static constexpr int NDT = HD / 16;                 // 16-channel output tiles
  static constexpr int VF = sizeof(T) == 2 ? 1 : 2;   // V fragments per channel per block
  u32x4 k[2][FR];
  u32x4 v[NDT][VF];
};

template <typename T, int HD>
__device__ __forceinline__ void load_block(KVBlock<T, HD>& b, const T* K, const T* V, int kb,
                                           int k_hi, int r, int grp) {
  using KB = KVBlock<T, HD>;
  // Fragment f of lane group g holds head-dim channels [4*EPF*f + EPF*g, +EPF):
  // one load instruction reads 64 contiguous bytes of 16 key rows.
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int key = kb + key_of<T>(t, r);
    const bool ok = key < k_hi;
    const T* kp = K + (size_t)key * HD + grp * KB::EPF;
#pragma unroll
    for (int f = 0; f < KB::FR; ++f) b.k[t][f] = ok ? ld16(kp + f * 4 * KB::EPF) : zero16();
  }
  const T* vb = V + (size_t)(kb / kKeyBlock) * HD * kKeyBlock;
  const bool tail = kb + 32 > k_hi;
#pragma unroll
  for (int dt = 0; dt < KB::NDT; ++dt) {
    const int d = 16 * dt + r;
#pragma unroll
    for (int u = 0; u < KB::VF; ++u) {
      const int koff = (sizeof(T) == 2) ? 8 * grp : 16 * u + 4 * grp;
      u32x4 x = ld16(vb + d * kKeyBlock + koff);
      if (tail) x = keep_first<T>(x, k_hi - (kb + koff));
      b.v[dt][u] = x;
    }
  }
}

template <typename T, int HD>
__global__ __launch_bounds__(512) void attn_partial_kernel(AttnArgs p) {
  using KB = KVBlock<T, HD>;
  constexpr int EPF = KB::EPF, FR = KB::FR, NDT = KB::NDT;
  const int lane = threadIdx.x & 63, j = threadIdx.x >> 6;
  const int r = lane & 15, grp = lane >> 4;
  const int c = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int G = p.n_heads / p.n_kv_heads;
  const int h = g * G + j;

  const int n_keys = seq_keys(p, s);
  const int k_lo = c * p.chunk;
  if (k_lo >= n_keys) return;
  const int k_hi = min(n_keys, k_lo + p.chunk);
  const bool single = n_keys <= p.chunk;

  const size_t kvoff = (size_t)(s * p.n_kv_heads + g) * p.cap * HD;
  const T* K = reinterpret_cast<const T*>(p.k) + kvoff;
  const T* V = reinterpret_cast<const T*>(p.v) + kvoff;

  u32x4 qf[FR];  // same channel order as the K fragments
  {
    const T* qp = reinterpret_cast<const T*>(p.q) + (((size_t)s * p.n_heads + h) * 16 + r) * HD +
                  grp * EPF;
#pragma unroll
    for (int f = 0; f < FR; ++f) qf[f] = ld16(qp + f * 4 * EPF);
  }

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto process = [&](const KB& b, int kb) {
    f32x4 st[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      st[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int f = 0; f < FR; ++f) st[t] = mfma_frag<T>(b.k[t][f], qf[f], st[t]);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = kb + key_of<T>(t, 4 * grp + i);
        const float v = key < k_hi ? st[t][i] * p.scale_log2 : -INFINITY;
        st[t][i] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // Every block holds at least one valid key, so m_new is finite.
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pv = exp2f(st[t][i] - m_new);
        st[t][i] = pv;
        psum += pv;
      }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;
    if constexpr (sizeof(T) == 2) {
      bf16x8 pb;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) pb[4 * t + i] = (bf16)st[t][i];
      const u32x4 pf = __builtin_bit_cast(u32x4, pb);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[dt] = mfma_frag<T>(b.v[dt][0], pf, o[dt]);
    } else {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const u32x4 pf = __builtin_bit_cast(u32x4, st[t]);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[dt] = mfma_frag<T>(b.v[dt][t], pf, o[dt]);
      }
    }
  };

  if constexpr (sizeof(T) == 2 || HD == 64) {
    // Two blocks in flight: the next block's K/V loads while this one is used.
    KB b0, b1;
    load_block<T, HD>(b0, K, V, k_lo, k_hi, r, grp);
    for (int kb = k_lo; kb < k_hi; kb += 64) {
      const bool has1 = kb + 32 < k_hi;
      if (has1) load_block<T, HD>(b1, K, V, kb + 32, k_hi, r, grp);
      process(b0, kb);
      if (has1) {
        if (kb + 64 < k_hi) load_block<T, HD>(b0, K, V, kb + 64, k_hi, r, grp);
        process(b1, kb + 32);
      }
    }
  } else {
    // fp32 at head_dim 128: one block of fragments already fills the registers.
    for (int kb = k_lo; kb < k_hi; kb += 32) {
      KB b0;
      load_block<T, HD>(b0, K, V, kb, k_hi, r, grp);
      process(b0, kb);
    }
  }

  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (single) {
    // The whole sequence was in this chunk: normalise and write the output.
    if (r < p.block) {
      // Four consecutive channels per lane and tile: contiguous in the tiled output.
      const float inv = 1.0f / l_run;
      T* out = reinterpret_cast<T*>(p.out);
      const int row = s * p.block + r;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        T* dst = out + tiled_index<T>(row, h * HD + 16 * dt + 4 * grp, p.out_nck);
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[i] = from_f32<T>(o[dt][i] * inv);
      }
    }
    return;
  }
  const size_t item = ((size_t)(s * p.n_kv_heads + g) * p.max_chunks + c) * G + j;
  if (grp == 0) {
    p.part_ml[(item * 16 + r) * 2 + 0] = m_run;
    p.part_ml[(item * 16 + r) * 2 + 1] = l_run;
  }
  float* po = p.part_o + item * HD * 16;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) po[(16 * dt + 4 * grp + i) * 16 + r] = o[dt][i];
}

// Merge of the chunk partials of one (query head, sequence, 16-channel slice).
// Thread (q, cg) owns query row q and the chunks c = cg, cg + 16, ...: it
// reduces the row's running max and sum over its chunks, the 16 threads of a
// row combine them through LDS, then each thread accumulates its chunks'
// weighted partial outputs for the slice's 16 channels and LDS sums the 16
// chunk groups. Every thread's loads are independent of each other.
template <typename T, int HD>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs p) {
  __shared__ float red_m[16][17], red_l[16][17];
  __shared__ float red_o[16][16][17];
  const int h = blockIdx.x, s = blockIdx.y, slice = blockIdx.z;
  const int G = p.n_heads / p.n_kv_heads;
  const int g = h / G, j = h % G;
  const int n_keys = seq_keys(p, s);
  const int nch = (n_keys + p.chunk - 1) / p.chunk;
  if (nch <= 1) return;  // written by the partial kernel
  const int t = threadIdx.x, q = t & 15, cg = t >> 4;
  const size_t item0 = (size_t)(s * p.n_kv_heads + g) * p.max_chunks * G + j;
  float m = -INFINITY;
  for (int c = cg; c < nch; c += 16) m = fmaxf(m, p.part_ml[((item0 + (size_t)c * G) * 16 + q) * 2]);
  red_m[q][cg] = m;
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int k = 0; k < 16; ++k) M = fmaxf(M, red_m[q][k]);
  float l = 0.f;
  for (int c = cg; c < nch; c += 16) {
    const float* ml = p.part_ml + ((item0 + (size_t)c * G) * 16 + q) * 2;
    l += ml[1] * exp2f(ml[0] - M);
  }
  red_l[q][cg] = l;
  __syncthreads();
  float L = 0.f;
#pragma unroll
  for (int k = 0; k < 16; ++k) L += red_l[q][k];
  const float inv = 1.0f / L;
  float acc[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) acc[k] = 0.f;
  for (int c = cg; c < nch; c += 16) {
    const size_t it = item0 + (size_t)c * G;
    const float w = exp2f(p.part_ml[(it * 16 + q) * 2] - M) * inv;
    const float* po = p.part_o + (it * HD + 16 * slice) * 16 + q;
#pragma unroll
    for (int k = 0; k < 16; ++k) acc[k] += po[k * 16] * w;
  }
#pragma unroll
  for (int k = 0; k < 16; ++k) red_o[k][cg][q] = acc[k];
  __syncthreads();
  // thread (q, d = cg) sums the 16 chunk groups of channel 16*slice + d
  if (q < p.block) {
    float o = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) o += red_o[cg][k][q];
    T* out = reinterpret_cast<T*>(p.out);
    out[tiled_index<T>(s * p.block + q, h * HD + 16 * slice + cg, p.out_nck)] = from_f32<T>(o);
  }
}

template <typename T, int HD>
static hipError_t launch_hd(const AttnArgs& a, hipStream_t st) {
  const int G = a.n_heads / a.n_kv_heads;
  dim3 grid(a.max_chunks, a.n_kv_heads, a.batch);
  hipLaunchKernelGGL((attn_partial_kernel<T, HD>), grid, dim3(64 * G), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_chunks <= 1) return e;
  prof_end(st);
  prof_begin(DFLASH_K_ATTN_COMBINE, 0.0, 0.0, st);
  hipLaunchKernelGGL((attn_combine_kernel<T, HD>), dim3(a.n_heads, a.batch, HD / 16), dim3(256), 0,
                     st, a);
  return hipGetLastError();
}

hipError_t launch_attention(int dtype, const AttnArgs& a, hipStream_t st) {
  if (a.n_heads / a.n_kv_heads > 8) return hipErrorInvalidValue;
  if (dtype == DFLASH_BF16) {
    if (a.head_dim == 128) return launch_hd<bf16, 128>(a, st);
    if (a.head_dim == 64) return launch_hd<bf16, 64>(a, st);
  } else {
    if (a.head_dim == 128) return launch_hd<float, 128>(a, st);
    if (a.head_dim == 64) return launch_hd<float, 64>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace dflash
