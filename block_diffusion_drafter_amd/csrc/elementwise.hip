// Row-wise and bookkeeping kernels of the drafter pass: RMSNorm, the block
// embedding, per-head q/k RMSNorm + rotary embedding + K/V cache scatter,
// the cross-tile argmax reduction, greedy acceptance and the context-length
// update. All are small next to the weight and cache streams; they are written
// for coalesced row access and one pass over their data.
#include "common.h"
#include "internal.h"

namespace dflash {

__device__ __forceinline__ float block_sum_256(float v, float* sh) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) t += sh[i];
  return t;
}

// y[r] = x[src(r)] / sqrt(mean(x^2) + eps) * gain, statistics in fp32.
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* x, int64_t xs, const T* gain,
                                                      T* y, int64_t ys, int d, float eps, int rpg,
                                                      int grp_stride, int grp_off) {
  __shared__ float sh[4];
  const int r = blockIdx.x;
  const int64_t src = (int64_t)(r / rpg) * grp_stride + grp_off + r % rpg;
  const float* xr = x + src * xs;
  T* yr = y + (int64_t)r * ys;
  float ss = 0.f;
  for (int k = threadIdx.x; k < d; k += blockDim.x) ss += xr[k] * xr[k];
  ss = block_sum_256(ss, sh);
  const float inv = rsqrtf(ss / (float)d + eps);
  for (int k = threadIdx.x; k < d; k += blockDim.x) yr[k] = from_f32<T>(xr[k] * inv * to_f32(gain[k]));
}

hipError_t launch_rmsnorm(int dtype, const float* x, int64_t x_stride, const void* gain, void* y,
                          int64_t y_stride, int rows, int d, float eps, int rpg, int grp_stride,
                          int grp_off, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  if (dtype == DFLASH_BF16)
    hipLaunchKernelGGL(rmsnorm_kernel<bf16>, dim3(rows), dim3(256), 0, st, x, x_stride,
                       (const bf16*)gain, (bf16*)y, y_stride, d, eps, rpg, grp_stride, grp_off);
  else
    hipLaunchKernelGGL(rmsnorm_kernel<float>, dim3(rows), dim3(256), 0, st, x, x_stride,
                       (const float*)gain, (float*)y, y_stride, d, eps, rpg, grp_stride, grp_off);
  return hipGetLastError();
}

// x[s*B + i] = E[i == 0 ? anchor[s] : mask] (input_embedding_scale 1).
template <typename T>
__global__ __launch_bounds__(256) void embed_kernel(const T* E, const int32_t* anchor, int block,
                                                    int d, int vocab, int mask_id, float* x,
                                                    int32_t* dev_status) {
  const int row = blockIdx.x, s = row / block, i = row % block;
  int id = i == 0 ? anchor[s] : mask_id;
  if (id < 0 || id >= vocab) {
    if (threadIdx.x == 0 && dev_status) atomicOr(dev_status, DFLASH_DEV_TOKEN);
    id = id < 0 ? 0 : vocab - 1;
  }
  const T* e = E + (int64_t)id * d;
  float* xr = x + (int64_t)row * d;
  for (int k = threadIdx.x; k < d; k += blockDim.x) xr[k] = to_f32(e[k]);
}

hipError_t launch_embed(int dtype, const void* embed, const int32_t* anchor, int batch, int block,
                        int d, int vocab, int mask_id, float* x, int32_t* dev_status,
                        hipStream_t st) {
  if (dtype == DFLASH_BF16)
    hipLaunchKernelGGL(embed_kernel<bf16>, dim3(batch * block), dim3(256), 0, st,
                       (const bf16*)embed, anchor, block, d, vocab, mask_id, x, dev_status);
  else
    hipLaunchKernelGGL(embed_kernel<float>, dim3(batch * block), dim3(256), 0, st,
                       (const float*)embed, anchor, block, d, vocab, mask_id, x, dev_status);
  return hipGetLastError();
}

// One wave normalises one head vector: lane l owns channels l and l + HD/2,
// which is exactly one rotary pair.
template <typename T, int HD>
__device__ __forceinline__ void norm_rope_head(float x0, float x1, const T* gain, float eps,
                                               float theta, int pos, int lane, float& o0,
                                               float& o1) {
  constexpr int HALF = HD / 2;
  const float ss = wave_sum(x0 * x0 + x1 * x1);
  const float inv = rsqrtf(ss / (float)HD + eps);
  float y0 = 0.f, y1 = 0.f;
  if (lane < HALF) {
    y0 = x0 * inv * to_f32(gain[lane]);
    y1 = x1 * inv * to_f32(gain[lane + HALF]);
  }
  if (theta > 0.f && lane < HALF) {
    // Angle in double: positions reach tens of thousands of radians.
    const double inv_freq = pow((double)theta, -2.0 * (double)lane / (double)HD);
    const double ang = (double)pos * inv_freq;
    double sn, cs;
    sincos(ang, &sn, &cs);
    const float c = (float)cs, s = (float)sn;
    o0 = y0 * c - y1 * s;
    o1 = y1 * c + y0 * s;
  } else {
    o0 = y0;
    o1 = y1;
  }
}

template <typename T, int HD>
__device__ __forceinline__ void store_v(T* vbase, int pos, int lane, float x0, float x1) {
  constexpr int HALF = HD / 2;
  if (lane < HALF) {
    T* blk = vbase + (size_t)(pos / kKeyBlock) * HD * kKeyBlock + (pos % kKeyBlock);
    blk[(size_t)lane * kKeyBlock] = from_f32<T>(x0);
    blk[(size_t)(lane + HALF) * kKeyBlock] = from_f32<T>(x1);
  }
}

// Forward mode: grid (Hq + 2*Hkv, batch*16), one wave per (head, block slot).
template <typename T, int HD>
__global__ __launch_bounds__(64) void norm_rope_fwd_kernel(NormRopeArgs p) {
  constexpr int HALF = HD / 2;
  const int head = blockIdx.x, slot = blockIdx.y, s = slot / 16, i = slot % 16;
  const int lane = threadIdx.x;
  const int Hq = p.n_heads, Hkv = p.n_kv_heads;
  if (head < Hq) {
    T* qo = reinterpret_cast<T*>(p.q_out) + (((size_t)s * Hq + head) * 16 + i) * HD;
    if (i >= p.block) {
      if (lane < HALF) {
        qo[lane] = from_f32<T>(0.f);
        qo[lane + HALF] = from_f32<T>(0.f);
      }
      return;
    }
  } else if (i >= p.block) {
    return;
  }
  const int m = s * p.block + i;
  const float* src = p.src + (int64_t)m * p.src_stride + (int64_t)head * HD;
  const float x0 = lane < HALF ? src[lane] : 0.f;
  const float x1 = lane < HALF ? src[lane + HALF] : 0.f;
  int cl = p.ctx_len[s];
  cl = cl < 0 ? 0 : cl;
  const int pos = cl + i;
  const bool in_cap = pos < p.cap;
  if (head >= Hq + Hkv) {
    if (!in_cap) {
      if (lane == 0 && p.dev_status) atomicOr(p.dev_status, DFLASH_DEV_CAPACITY);
      return;
    }
    const int g = head - Hq - Hkv;
    T* vbase = reinterpret_cast<T*>(p.v_cache) + (size_t)(s * Hkv + g) * p.cap * HD;
    store_v<T, HD>(vbase, pos, lane, x0, x1);
    return;
  }
  const bool is_q = head < Hq;
  const T* gain = reinterpret_cast<const T*>(is_q ? p.q_norm[0] : p.k_norm[0]);
  float o0, o1;
  norm_rope_head<T, HD>(x0, x1, gain, p.eps, p.rope_theta, pos, lane, o0, o1);
  if (lane >= HALF) return;
  if (is_q) {
    T* qo = reinterpret_cast<T*>(p.q_out) + (((size_t)s * Hq + head) * 16 + i) * HD;
    qo[lane] = from_f32<T>(o0);
    qo[lane + HALF] = from_f32<T>(o1);
  } else {
    if (!in_cap) {
      if (lane == 0 && p.dev_status) atomicOr(p.dev_status, DFLASH_DEV_CAPACITY);
      return;
    }
    const int g = head - Hq;
    T* kr = reinterpret_cast<T*>(p.k_cache) + ((size_t)(s * Hkv + g) * p.cap + pos) * HD;
    kr[lane] = from_f32<T>(o0);
    kr[lane + HALF] = from_f32<T>(o1);
  }
}

// Append mode: grid (n_layers * 2 * Hkv, n_tok); column c = layer * 2*Hkv + h,
// h < Hkv a key head, h >= Hkv a value head.
template <typename T, int HD>
__global__ __launch_bounds__(64) void norm_rope_append_kernel(NormRopeArgs p) {
  constexpr int HALF = HD / 2;
  const int col = blockIdx.x, row = blockIdx.y, lane = threadIdx.x;
  const int Hkv = p.n_kv_heads;
  const int l = col / (2 * Hkv), hh = col % (2 * Hkv);
  int s = -1;
  for (int t = 0; t < p.batch; ++t) {
    if (p.cu_new[t] <= row && row < p.cu_new[t + 1]) {
      s = t;
      break;
    }
  }
  if (s < 0) {
    if (lane == 0 && p.dev_status) atomicOr(p.dev_status, DFLASH_DEV_OFFSETS);
    return;
  }
  int cl = p.ctx_len[s];
  cl = cl < 0 ? 0 : cl;
  const int pos = cl + (row - p.cu_new[s]);
  if (pos >= p.cap) {
    if (lane == 0 && p.dev_status) atomicOr(p.dev_status, DFLASH_DEV_CAPACITY);
    return;
  }
  const float* src = p.src + (int64_t)row * p.src_stride + (int64_t)col * HD;
  const float x0 = lane < HALF ? src[lane] : 0.f;
  const float x1 = lane < HALF ? src[lane + HALF] : 0.f;
  const size_t layer_stride = (size_t)p.cache_batch * Hkv * p.cap * HD;
  if (hh >= Hkv) {
    const int g = hh - Hkv;
    T* vbase = reinterpret_cast<T*>(p.v_cache) + l * layer_stride + (size_t)(s * Hkv + g) * p.cap * HD;
    store_v<T, HD>(vbase, pos, lane, x0, x1);
    return;
  }
  const int g = hh;
  float o0, o1;
  norm_rope_head<T, HD>(x0, x1, reinterpret_cast<const T*>(p.k_norm[l]), p.eps, p.rope_theta, pos,
                        lane, o0, o1);
  if (lane >= HALF) return;
  T* kr = reinterpret_cast<T*>(p.k_cache) + l * layer_stride + ((size_t)(s * Hkv + g) * p.cap + pos) * HD;
  kr[lane] = from_f32<T>(o0);
  kr[lane + HALF] = from_f32<T>(o1);
}

template <int MODE>
static hipError_t launch_nr(int dtype, const NormRopeArgs& a, dim3 grid, hipStream_t st) {
  const bool bf = dtype == DFLASH_BF16;
  if (a.head_dim == 128) {
    if (MODE == 0) {
      if (bf) hipLaunchKernelGGL((norm_rope_fwd_kernel<bf16, 128>), grid, dim3(64), 0, st, a);
      else hipLaunchKernelGGL((norm_rope_fwd_kernel<float, 128>), grid, dim3(64), 0, st, a);
    } else {
      if (bf) hipLaunchKernelGGL((norm_rope_append_kernel<bf16, 128>), grid, dim3(64), 0, st, a);
      else hipLaunchKernelGGL((norm_rope_append_kernel<float, 128>), grid, dim3(64), 0, st, a);
    }
  } else if (a.head_dim == 64) {
    if (MODE == 0) {
      if (bf) hipLaunchKernelGGL((norm_rope_fwd_kernel<bf16, 64>), grid, dim3(64), 0, st, a);
      else hipLaunchKernelGGL((norm_rope_fwd_kernel<float, 64>), grid, dim3(64), 0, st, a);
    } else {
      if (bf) hipLaunchKernelGGL((norm_rope_append_kernel<bf16, 64>), grid, dim3(64), 0, st, a);
      else hipLaunchKernelGGL((norm_rope_append_kernel<float, 64>), grid, dim3(64), 0, st, a);
    }
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_norm_rope_forward(int dtype, const NormRopeArgs& a, hipStream_t st) {
  return launch_nr<0>(dtype, a, dim3(a.n_heads + 2 * a.n_kv_heads, a.batch * 16), st);
}

hipError_t launch_norm_rope_append(int dtype, const NormRopeArgs& a, hipStream_t st) {
  if (a.n_tok <= 0) return hipSuccess;
  return launch_nr<1>(dtype, a, dim3(a.n_layers * 2 * a.n_kv_heads, a.n_tok), st);
}

__global__ __launch_bounds__(256) void argmax_reduce_kernel(const unsigned long long* amax,
                                                            int64_t stride, int n_tiles,
                                                            int32_t* tokens) {
  __shared__ unsigned long long sh[256];
  const int row = blockIdx.x;
  unsigned long long best = 0ull;
  for (int t = threadIdx.x; t < n_tiles; t += blockDim.x) {
    const unsigned long long k = amax[(int64_t)row * stride + t];
    best = k > best ? k : best;
  }
  sh[threadIdx.x] = best;
  __syncthreads();
  for (int o = blockDim.x / 2; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) {
      const unsigned long long k = sh[threadIdx.x + o];
      if (k > sh[threadIdx.x]) sh[threadIdx.x] = k;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) tokens[row] = (int32_t)argmax_index(sh[0]);
}

hipError_t launch_argmax_reduce(const unsigned long long* amax, int64_t stride, int n_tiles,
                                int rows, int32_t* tokens, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(argmax_reduce_kernel, dim3(rows), dim3(256), 0, st, amax, stride, n_tiles,
                     tokens);
  return hipGetLastError();
}

__global__ void accept_kernel(const int32_t* drafts, const int32_t* targets, int batch, int block,
                              int32_t* accept_len, int32_t* bonus, int32_t* anchor_out) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= batch) return;
  const int m = block - 1;
  const int32_t* d = drafts + (int64_t)s * m;
  const int32_t* t = targets + (int64_t)s * block;
  int a = 0;
  while (a < m && d[a] == t[a]) ++a;
  accept_len[s] = a;
  bonus[s] = t[a];
  if (anchor_out) anchor_out[s] = t[a];
}

hipError_t launch_accept(const int32_t* drafts, const int32_t* targets, int batch, int block,
                         int32_t* accept_len, int32_t* bonus, int32_t* anchor_out,
                         hipStream_t st) {
  if (batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(accept_kernel, dim3((batch + 63) / 64), dim3(64), 0, st, drafts, targets,
                     batch, block, accept_len, bonus, anchor_out);
  return hipGetLastError();
}

__global__ void ctx_len_add_kernel(int32_t* ctx_len, const int32_t* cu_new, int batch, int n_tok,
                                   int cap, int32_t* dev_status) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s == 0 && (cu_new[0] != 0 || cu_new[batch] != n_tok) && dev_status)
    atomicOr(dev_status, DFLASH_DEV_OFFSETS);
  if (s >= batch) return;
  int n = cu_new[s + 1] - cu_new[s];
  if (n < 0) {
    if (dev_status) atomicOr(dev_status, DFLASH_DEV_OFFSETS);
    n = 0;
  }
  int cl = ctx_len[s];
  cl = cl < 0 ? 0 : cl;
  int nl = cl + n;
  if (nl > cap) {
    if (dev_status) atomicOr(dev_status, DFLASH_DEV_CAPACITY);
    nl = cap;
  }
  ctx_len[s] = nl;
}

hipError_t launch_ctx_len_add(int32_t* ctx_len, const int32_t* cu_new, int batch, int n_tok,
                              int cap, int32_t* dev_status, hipStream_t st) {
  hipLaunchKernelGGL(ctx_len_add_kernel, dim3((batch + 63) / 64), dim3(64), 0, st, ctx_len, cu_new,
                     batch, n_tok, cap, dev_status);
  return hipGetLastError();
}

}  // namespace dflash
