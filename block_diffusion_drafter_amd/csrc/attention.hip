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
  constexpr int SPAN = HD / 4;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int key = kb + key_of<T>(t, r);
    const bool ok = key < k_hi;
    const T* kp = K + (size_t)key * HD + grp * SPAN;
#pragma unroll
    for (int f = 0; f < KB::FR; ++f) b.k[t][f] = ok ? ld16(kp + f * KB::EPF) : zero16();
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
  constexpr int SPAN = HD / 4;
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

  u32x4 qf[FR];
  {
    const T* qp = reinterpret_cast<const T*>(p.q) + (((size_t)s * p.n_heads + h) * 16 + r) * HD +
                  grp * SPAN;
#pragma unroll
    for (int f = 0; f < FR; ++f) qf[f] = ld16(qp + f * EPF);
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
      const float inv = 1.0f / l_run;
      T* out = reinterpret_cast<T*>(p.out) + ((size_t)s * p.block + r) * p.n_heads * HD +
               (size_t)h * HD;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) out[16 * dt + 4 * grp + i] = from_f32<T>(o[dt][i] * inv);
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

// One workgroup per (query head, sequence). Thread t owns query row t % 16 and
// channels t / 16 + 16 k; the chunk weights exp2(m_c - M) / L are computed once
// into LDS, and every thread's chunk loop issues independent loads.
template <typename T, int HD>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs p) {
  extern __shared__ float wsh[];  // [nch][16]: m_c, then the chunk weight
  __shared__ float lsh[16 * 16];
  const int h = blockIdx.x, s = blockIdx.y;
  const int G = p.n_heads / p.n_kv_heads;
  const int g = h / G, j = h % G;
  const int n_keys = seq_keys(p, s);
  const int nch = (n_keys + p.chunk - 1) / p.chunk;
  if (nch <= 1) return;  // written by the partial kernel
  const int t = threadIdx.x, q = t & 15, part = t >> 4;
  const size_t item0 = (size_t)(s * p.n_kv_heads + g) * p.max_chunks * G + j;
  // 1. every chunk's running max into LDS
  for (int idx = t; idx < nch * 16; idx += 256) {
    const int c = idx >> 4, qq = idx & 15;
    wsh[idx] = p.part_ml[((item0 + (size_t)c * G) * 16 + qq) * 2];
  }
  __syncthreads();
  // 2. the row's global max; 3. its sum, split over the 16 threads of the row
  float M = -INFINITY;
  for (int c = 0; c < nch; ++c) M = fmaxf(M, wsh[c * 16 + q]);
  float L = 0.f;
  for (int c = part; c < nch; c += 16)
    L += p.part_ml[((item0 + (size_t)c * G) * 16 + q) * 2 + 1] * exp2f(wsh[c * 16 + q] - M);
  lsh[part * 16 + q] = L;
  __syncthreads();
  L = 0.f;
#pragma unroll
  for (int k = 0; k < 16; ++k) L += lsh[k * 16 + q];
  const float inv = 1.0f / L;
  // 4. one thread per row turns the chunk maxima into weights exp2(m_c - M) / L
  if (part == 0)
    for (int c = 0; c < nch; ++c) wsh[c * 16 + q] = exp2f(wsh[c * 16 + q] - M) * inv;
  __syncthreads();
  if (q >= p.block) return;
  constexpr int PER = HD / 16;
  float acc[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) acc[k] = 0.f;
#pragma unroll 2
  for (int c = 0; c < nch; ++c) {
    const float wgt = wsh[c * 16 + q];
    const float* po = p.part_o + (item0 + (size_t)c * G) * HD * 16;
#pragma unroll
    for (int k = 0; k < PER; ++k) acc[k] += po[(part + 16 * k) * 16 + q] * wgt;
  }
  T* out = reinterpret_cast<T*>(p.out) + ((size_t)s * p.block + q) * p.n_heads * HD + (size_t)h * HD;
#pragma unroll
  for (int k = 0; k < PER; ++k) out[part + 16 * k] = from_f32<T>(acc[k]);
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
  const size_t lds = (size_t)a.max_chunks * 16 * sizeof(float);
  hipLaunchKernelGGL((attn_combine_kernel<T, HD>), dim3(a.n_heads, a.batch), dim3(256), lds, st, a);
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
