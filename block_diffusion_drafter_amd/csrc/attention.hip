// KV-injected attention of the draft block over [cached context ; block] keys.
//
// The block's queries (B <= 16 rows per head) attend non-causally to every
// cached context position of their sequence plus the block's own keys, which
// the QKV step has already staged in the cache's scratch positions
// [ctx_len, ctx_len + B). With 16 queries per head over thousands of keys the
// work is a stream of the K/V cache, so it is split over key chunks:
//
//   attn_partial: one wave per (sequence, KV head, key chunk). The wave packs
//     all query heads that share the KV head (GQA group x 16 rows) and loads
//     each K/V position once. Scores are computed transposed, S^T = K Q^T
//     (keys as MFMA rows, queries as columns), and the output likewise,
//     O^T = V^T P^T, so each lane owns one query column: the online-softmax
//     running max/sum are per-lane values plus a two-step shuffle across the
//     four lane groups. P leaves the S^T accumulator already in the layout
//     the next MFMA's B operand needs (the key order inside a 32-key block is
//     permuted to make that so). V is stored channel-major inside 32-position
//     blocks, so each lane's V fragment is one 16-byte load.
//   attn_combine: merges the chunks' (max, sum, unnormalised O) per query row.
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
      unsigned mask = (e0 < nvalid ? 0x0000FFFFu : 0u) | (e0 + 1 < nvalid ? 0xFFFF0000u : 0u);
      v[w] &= mask;
    }
  } else {
#pragma unroll
    for (int w = 0; w < 4; ++w)
      if (w >= nvalid) v[w] = 0u;
  }
  return v;
}

template <typename T, int HD, int GH>
__global__ __launch_bounds__(64) void attn_partial_kernel(AttnArgs p) {
  constexpr int EPF = 16 / (int)sizeof(T);
  constexpr int SPAN = HD / 4;          // head-dim elements per lane group
  constexpr int FR = SPAN / EPF;        // 16-byte fragments per lane per key row
  constexpr int NDT = HD / 16;          // 16-channel tiles of the output
  constexpr int VF = sizeof(T) == 2 ? 1 : 2;  // V fragments per channel per 32 keys
  const int lane = threadIdx.x, r = lane & 15, grp = lane >> 4;
  const int c = blockIdx.x, g = blockIdx.y, s = blockIdx.z;

  int cl = p.ctx_len[s];
  cl = cl < 0 ? 0 : cl;
  const int n_keys = min(cl + p.block, p.cap);
  const int k_lo = c * p.chunk;
  if (k_lo >= n_keys) return;
  const int k_hi = min(n_keys, k_lo + p.chunk);

  const size_t kvoff = (size_t)(s * p.n_kv_heads + g) * p.cap * HD;
  const T* K = reinterpret_cast<const T*>(p.k) + kvoff;
  const T* V = reinterpret_cast<const T*>(p.v) + kvoff;

  u32x4 qf[GH][FR];
#pragma unroll
  for (int j = 0; j < GH; ++j) {
    const T* qp = reinterpret_cast<const T*>(p.q) +
                  (((size_t)s * p.n_heads + g * GH + j) * 16 + r) * HD + grp * SPAN;
#pragma unroll
    for (int f = 0; f < FR; ++f) qf[j][f] = ld16(qp + f * EPF);
  }

  float m_run[GH], l_run[GH];
  f32x4 o[GH][NDT];
#pragma unroll
  for (int j = 0; j < GH; ++j) {
    m_run[j] = -INFINITY;
    l_run[j] = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[j][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  for (int kb = k_lo; kb < k_hi; kb += 32) {
    u32x4 kf[2][FR];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int key = kb + key_of<T>(t, r);
      const bool ok = key < k_hi;
      const T* kp = K + (size_t)key * HD + grp * SPAN;
#pragma unroll
      for (int f = 0; f < FR; ++f) kf[t][f] = ok ? ld16(kp + f * EPF) : zero16();
    }
    u32x4 vf[NDT][VF];
    const T* vb = V + (size_t)(kb / kKeyBlock) * HD * kKeyBlock;
    const bool tail = kb + 32 > k_hi;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const int d = 16 * dt + r;
#pragma unroll
      for (int u = 0; u < VF; ++u) {
        const int koff = (sizeof(T) == 2) ? 8 * grp : 16 * u + 4 * grp;
        u32x4 x = ld16(vb + d * kKeyBlock + koff);
        if (tail) x = keep_first<T>(x, k_hi - (kb + koff));
        vf[dt][u] = x;
      }
    }

#pragma unroll
    for (int j = 0; j < GH; ++j) {
      f32x4 st[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        st[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int f = 0; f < FR; ++f) st[t] = mfma_frag<T>(kf[t][f], qf[j][f], st[t]);
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
      const float m_new = fmaxf(m_run[j], mx);
      const float alpha = exp2f(m_run[j] - m_new);
      m_run[j] = m_new;
      float psum = 0.f;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pv = exp2f(st[t][i] - m_new);
          st[t][i] = pv;
          psum += pv;
        }
      l_run[j] = l_run[j] * alpha + psum;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[j][dt] *= alpha;
      if constexpr (sizeof(T) == 2) {
        bf16x8 pb;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) pb[4 * t + i] = (bf16)st[t][i];
        const u32x4 pf = __builtin_bit_cast(u32x4, pb);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[j][dt] = mfma_frag<T>(vf[dt][0], pf, o[j][dt]);
      } else {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const u32x4 pf = __builtin_bit_cast(u32x4, st[t]);
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) o[j][dt] = mfma_frag<T>(vf[dt][t], pf, o[j][dt]);
        }
      }
    }
  }

  const size_t item = ((size_t)(s * p.n_kv_heads + g) * p.max_chunks + c) * GH;
#pragma unroll
  for (int j = 0; j < GH; ++j) {
    float l = l_run[j];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (grp == 0) {
      p.part_ml[((item + j) * 16 + r) * 2 + 0] = m_run[j];
      p.part_ml[((item + j) * 16 + r) * 2 + 1] = l;
    }
    float* po = p.part_o + (item + j) * HD * 16;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) po[(16 * dt + 4 * grp + i) * 16 + r] = o[j][dt][i];
  }
}

template <typename T, int HD>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs p) {
  const int h = blockIdx.x, s = blockIdx.y;
  const int G = p.n_heads / p.n_kv_heads;
  const int g = h / G, j = h % G;
  const int q = threadIdx.x & 15, dpart = threadIdx.x >> 4;
  if (q >= p.block) return;
  int cl = p.ctx_len[s];
  cl = cl < 0 ? 0 : cl;
  const int n_keys = min(cl + p.block, p.cap);
  const int nch = (n_keys + p.chunk - 1) / p.chunk;
  const size_t item0 = (size_t)(s * p.n_kv_heads + g) * p.max_chunks * G + j;
  float M = -INFINITY;
  for (int c = 0; c < nch; ++c) M = fmaxf(M, p.part_ml[((item0 + (size_t)c * G) * 16 + q) * 2]);
  float L = 0.f;
  for (int c = 0; c < nch; ++c) {
    const float* ml = p.part_ml + ((item0 + (size_t)c * G) * 16 + q) * 2;
    L += ml[1] * exp2f(ml[0] - M);
  }
  const float inv = 1.0f / L;
  T* out = reinterpret_cast<T*>(p.out) + ((size_t)s * p.block + q) * p.n_heads * HD + (size_t)h * HD;
  for (int d = dpart; d < HD; d += 16) {
    float acc = 0.f;
    for (int c = 0; c < nch; ++c) {
      const size_t it = item0 + (size_t)c * G;
      acc += p.part_o[(it * HD + d) * 16 + q] * exp2f(p.part_ml[(it * 16 + q) * 2] - M);
    }
    out[d] = from_f32<T>(acc * inv);
  }
}

template <typename T, int HD>
static hipError_t launch_hd(const AttnArgs& a, hipStream_t st) {
  const int G = a.n_heads / a.n_kv_heads;
  dim3 grid(a.max_chunks, a.n_kv_heads, a.batch);
  switch (G) {
    case 1: hipLaunchKernelGGL((attn_partial_kernel<T, HD, 1>), grid, dim3(64), 0, st, a); break;
    case 2: hipLaunchKernelGGL((attn_partial_kernel<T, HD, 2>), grid, dim3(64), 0, st, a); break;
    case 4: hipLaunchKernelGGL((attn_partial_kernel<T, HD, 4>), grid, dim3(64), 0, st, a); break;
    case 8: hipLaunchKernelGGL((attn_partial_kernel<T, HD, 8>), grid, dim3(64), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  prof_end(st);
  prof_begin(DFLASH_K_ATTN_COMBINE, 0.0, 0.0, st);
  hipLaunchKernelGGL((attn_combine_kernel<T, HD>), dim3(a.n_heads, a.batch), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attention(int dtype, const AttnArgs& a, hipStream_t st) {
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
