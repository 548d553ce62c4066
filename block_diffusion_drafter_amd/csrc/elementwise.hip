// Row-wise and bookkeeping kernels of the drafter pass: RMSNorm, the block
// embedding, per-head q/k RMSNorm + rotary embedding + K/V cache scatter,
// the cross-tile argmax reduction, greedy acceptance and the context-length
// update. All are small next to the weight and cache streams; they are written
// for coalesced row access and one pass over their data.
#include <cmath>

#include "common.h"
#include "internal.h"

namespace dflash {

// Rows of a verified block that enter the context: the anchor and the accepted
// candidates, accept length + 1, with the length clamped to [0, block).
__device__ __forceinline__ int accepted_rows(int a, int block) {
  return (a < 0 ? 0 : (a >= block ? block - 1 : a)) + 1;
}

__device__ __forceinline__ float block_sum(float v, float* sh) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) t += sh[i];
  return t;
}

// Four consecutive gain values as fp32.
template <typename T> __device__ __forceinline__ float4 load4(const T* g);
template <> __device__ __forceinline__ float4 load4<float>(const float* g) {
  return *reinterpret_cast<const float4*>(g);
}
template <> __device__ __forceinline__ float4 load4<bf16>(const bf16* g) {
  const uint2 u = *reinterpret_cast<const uint2*>(g);
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                     __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
}

template <typename T> __device__ __forceinline__ void store4(T* y, float4 v);
template <> __device__ __forceinline__ void store4<float>(float* y, float4 v) {
  *reinterpret_cast<float4*>(y) = v;
}
template <> __device__ __forceinline__ void store4<bf16>(bf16* y, float4 v) {
  const bf16 b[4] = {(bf16)v.x, (bf16)v.y, (bf16)v.z, (bf16)v.w};
  *reinterpret_cast<uint2*>(y) = __builtin_bit_cast(uint2, b);
}

// RMSNorm of one row whose values thread t holds in v[u] (elements
// 4 (t + 256 u) .. +3, zero past d): one block reduction, one store pass.
// Output row yrow of y: row-major with stride ys when nck == 0, else tiled
// with nck chunks per row (four consecutive elements stay contiguous in both).
template <typename T, int VPT>
__device__ __forceinline__ void rmsnorm_regs(const float4 (&v)[VPT], const T* gain, T* y, int yrow,
                                             int64_t ys, int nck, int d, float eps, float* sh) {
  float ss = 0.f;
#pragma unroll
  for (int u = 0; u < VPT; ++u) ss += v[u].x * v[u].x + v[u].y * v[u].y + v[u].z * v[u].z + v[u].w * v[u].w;
  ss = block_sum(ss, sh);
  const float inv = rsqrtf(ss / (float)d + eps);
#pragma unroll
  for (int u = 0; u < VPT; ++u) {
    const int k = 4 * (threadIdx.x + u * blockDim.x);
    if (k < d) {
      const float4 g = load4<T>(gain + k);
      T* dst = nck ? y + tiled_index<T>(yrow, k, nck) : y + (int64_t)yrow * ys + k;
      store4<T>(dst, make_float4(v[u].x * inv * g.x, v[u].y * inv * g.y, v[u].z * inv * g.z,
                                 v[u].w * inv * g.w));
    }
  }
}

// One row per workgroup, VPT float4 per thread held in registers: one load
// pass, then rmsnorm_regs (d <= 4 * 256 * VPT).
template <typename T, int VPT>
__device__ __forceinline__ void rmsnorm_row(const float* xr, const T* gain, T* y, int yrow,
                                            int64_t ys, int nck, int d, float eps, float* sh) {
  float4 v[VPT];
#pragma unroll
  for (int u = 0; u < VPT; ++u) {
    const int k = 4 * (threadIdx.x + u * blockDim.x);
    v[u] = k < d ? *reinterpret_cast<const float4*>(xr + k) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  rmsnorm_regs<T, VPT>(v, gain, y, yrow, ys, nck, d, eps, sh);
}

// y[r] = x[src(r)] / sqrt(mean(x^2) + eps) * gain, statistics in fp32.
template <typename T, int VPT>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* x, int64_t xs, const T* gain,
                                                      T* y, int64_t ys, int nck, int d, float eps,
                                                      int rpg, int grp_stride, int grp_off) {
  __shared__ float sh[4];
  const int r = blockIdx.x;
  const int64_t src = (int64_t)(r / rpg) * grp_stride + grp_off + r % rpg;
  rmsnorm_row<T, VPT>(x + src * xs, gain, y, r, ys, nck, d, eps, sh);
}

template <typename T>
static void launch_rmsnorm_t(const float* x, int64_t xs, const T* g, T* y, int64_t ys, int nck,
                             int rows, int d, float eps, int rpg, int gs, int go, hipStream_t st) {
  const int vpt = (d + 1023) / 1024;
  dim3 grid(rows), block(256);
#define DF_NORM(V) \
  hipLaunchKernelGGL((rmsnorm_kernel<T, V>), grid, block, 0, st, x, xs, g, y, ys, nck, d, eps, rpg, gs, go)
  if (vpt <= 1) DF_NORM(1);
  else if (vpt <= 2) DF_NORM(2);
  else if (vpt <= 4) DF_NORM(4);
  else DF_NORM(8);
#undef DF_NORM
}

hipError_t launch_rmsnorm(int dtype, const float* x, int64_t x_stride, const void* gain, void* y,
                          int64_t y_stride, int y_nck, int rows, int d, float eps, int rpg,
                          int grp_stride, int grp_off, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  if (d > 8192 || d % 4) return hipErrorInvalidValue;
  if (dtype == DFLASH_BF16)
    launch_rmsnorm_t<bf16>(x, x_stride, (const bf16*)gain, (bf16*)y, y_stride, y_nck, rows, d, eps,
                           rpg, grp_stride, grp_off, st);
  else
    launch_rmsnorm_t<float>(x, x_stride, (const float*)gain, (float*)y, y_stride, y_nck, rows, d,
                            eps, rpg, grp_stride, grp_off, st);
  return hipGetLastError();
}

// End of a projection split over K, with the RMSNorm of its rows fused.
// RES (a residual projection): x[m] += sum of the ks fp32 partials of row m
// (slice order, then the residual, as splitk_reduce_kernel sums), and the
// RMSNorm of the updated row into y (tiled, nck chunks per row): the next
// projection's normalised input, without a second pass over x. !RES (a store
// projection whose output is only consumed normalised, the fusion): y[m] =
// RMSNorm(sum of the partials), row-major (row stride N) when nck is 0; x is
// neither read nor written.
template <int VPT, bool RES>
__global__ __launch_bounds__(256) void splitk_reduce_norm_kernel(const float* __restrict__ part,
                                                                 int ks, int M, int N,
                                                                 float* __restrict__ x, int64_t xs,
                                                                 const bf16* gain, bf16* y, int nck,
                                                                 float eps, int yblock) {
  constexpr int ZG = 4;  // slices loaded together (every load of a group before its adds)
  __shared__ float sh[4];
  const int m = blockIdx.x;
  const int64_t MN = (int64_t)M * N;
  float4 v[VPT], r[VPT];
#pragma unroll
  for (int u = 0; u < VPT; ++u) {
    const int k = 4 * (threadIdx.x + u * blockDim.x);
    r[u] = RES && k < N ? *reinterpret_cast<const float4*>(x + (int64_t)m * xs + k)
                        : make_float4(0.f, 0.f, 0.f, 0.f);
    v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  // Slices in order, ZG at a time (ks <= kMfmaMaxSplit).
  for (int z0 = 0; z0 < ks; z0 += ZG) {
    float4 q[VPT][ZG];
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int k = 4 * (threadIdx.x + u * blockDim.x);
      const float* pp = part + (int64_t)m * N + k;
#pragma unroll
      for (int z = 0; z < ZG; ++z)
        q[u][z] = k < N && z0 + z < ks ? *reinterpret_cast<const float4*>(pp + (z0 + z) * MN)
                                        : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < VPT; ++u)
#pragma unroll
      for (int z = 0; z < ZG; ++z) {
        if (z0 + z < ks) {
          v[u].x += q[u][z].x;
          v[u].y += q[u][z].y;
          v[u].z += q[u][z].z;
          v[u].w += q[u][z].w;
        }
      }
  }
  if constexpr (RES) {
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      float4 acc = v[u];
      acc.x += r[u].x;
      acc.y += r[u].y;
      acc.z += r[u].z;
      acc.w += r[u].w;
      v[u] = acc;
      const int k = 4 * (threadIdx.x + u * blockDim.x);
      if (k < N) *reinterpret_cast<float4*>(x + (int64_t)m * xs + k) = acc;
    }
  }
  // yblock > 0: only rows m % yblock != 0 are normalised, into y row
  // (m / yblock) * (yblock - 1) + m % yblock - 1 (a block's slots after its
  // anchor; the decision is the same for the whole workgroup).
  int yrow = m;
  if (yblock > 0) {
    if (m % yblock == 0) return;
    yrow = (m / yblock) * (yblock - 1) + m % yblock - 1;
  }
  rmsnorm_regs<bf16, VPT>(v, gain, y, yrow, N, nck, N, eps, sh);
}

hipError_t launch_splitk_reduce_norm(const float* part, int ks, int M, int N, float* x,
                                     int64_t x_stride, const void* gain, void* y, int y_nck,
                                     float eps, bool residual, int y_block, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  if (N > 8192 || N % 4 || x_stride % 4 || ks < 1 || ks > kMfmaMaxSplit) return hipErrorInvalidValue;
  const int vpt = (N + 1023) / 1024;
  dim3 grid(M), block(256);
#define DF_RN(V, R)                                                                               \
  hipLaunchKernelGGL((splitk_reduce_norm_kernel<V, R>), grid, block, 0, st, part, ks, M, N, x,   \
                     x_stride, (const bf16*)gain, (bf16*)y, y_nck, eps, y_block)
#define DF_RN2(V) \
  if (residual) DF_RN(V, true); else DF_RN(V, false)
  if (vpt <= 1) { DF_RN2(1); }
  else if (vpt <= 2) { DF_RN2(2); }
  else if (vpt <= 4) { DF_RN2(4); }
  else { DF_RN2(8); }
#undef DF_RN2
#undef DF_RN
  return hipGetLastError();
}

// x[s*B + i] = E[i == 0 ? anchor[s] : mask] (input_embedding_scale 1), and the
// first layer's pre-norm of that row, h = RMSNorm(x; gain), h tiled.
template <typename T, int VPT>
__global__ __launch_bounds__(256) void embed_kernel(const T* E, const int32_t* anchor, int block,
                                                    int d, int vocab, int mask_id, float* x,
                                                    const T* gain, float eps, T* h, int nck,
                                                    int32_t* dev_status, int32_t* arrivals) {
  __shared__ float sh[4];
  const int row = blockIdx.x, s = row / block, i = row % block;
  if (arrivals && i == 0 && threadIdx.x == 0) arrivals[s] = 0;
  int id = i == 0 ? anchor[s] : mask_id;
  if (id < 0 || id >= vocab) {
    if (threadIdx.x == 0 && dev_status) atomicOr(dev_status, DFLASH_DEV_TOKEN);
    id = id < 0 ? 0 : vocab - 1;
  }
  const T* e = E + (int64_t)id * d;
  float* xr = x + (int64_t)row * d;
  // The row stays in registers for its norm (each thread normalises the
  // elements it stored).
  float4 v[VPT];
#pragma unroll
  for (int u = 0; u < VPT; ++u) {
    const int k = 4 * (threadIdx.x + u * blockDim.x);
    v[u] = k < d ? load4<T>(e + k) : make_float4(0.f, 0.f, 0.f, 0.f);
    if (k < d) *reinterpret_cast<float4*>(xr + k) = v[u];
  }
  rmsnorm_regs<T, VPT>(v, gain, h, row, 0, nck, d, eps, sh);
}

hipError_t launch_embed(int dtype, const void* embed, const int32_t* anchor, int batch, int block,
                        int d, int vocab, int mask_id, float* x, const void* gain, float eps,
                        void* h, int32_t* dev_status, int32_t* arrivals, hipStream_t st) {
  if (d > 8192 || d % 4) return hipErrorInvalidValue;
  const int vpt = (d + 1023) / 1024;
  const int nck = tiled_nck(dtype, d);
  dim3 grid(batch * block), blk(256);
#define DF_EMBED(T, V)                                                                            \
  hipLaunchKernelGGL((embed_kernel<T, V>), grid, blk, 0, st, (const T*)embed, anchor, block, d,   \
                     vocab, mask_id, x, (const T*)gain, eps, (T*)h, nck, dev_status, arrivals)
  if (dtype == DFLASH_BF16) {
    if (vpt <= 1) DF_EMBED(bf16, 1); else if (vpt <= 2) DF_EMBED(bf16, 2);
    else if (vpt <= 4) DF_EMBED(bf16, 4); else DF_EMBED(bf16, 8);
  } else {
    if (vpt <= 1) DF_EMBED(float, 1); else if (vpt <= 2) DF_EMBED(float, 2);
    else if (vpt <= 4) DF_EMBED(float, 4); else DF_EMBED(float, 8);
  }
#undef DF_EMBED
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Per-head q/k RMSNorm + rotary embedding + K/V cache scatter.
//
// Rotary pairs: a head vector of HD channels is HD/2 pairs (channel c with
// c + HD/2). The angle pos * inv_freq is formed in double (positions reach
// tens of thousands of radians), reduced by 2 pi in double (Cody-Waite: 2 pi
// as the nearest double plus its remainder), and the reduced angle goes to
// the fp32 sincos.
//
// Forward (the block's rows, norm_rope_fwd_kernel): one workgroup per row
// and group of heads, many short workgroups (at batch 1 a handful of rows
// must still spread over the chip).
//
// Append (an append's new context rows, norm_rope_append_kernel): a
// workgroup takes a tile of up to 16 consecutive new rows of ONE sequence
// (stored at consecutive positions pos0 .. pos0 + nrows - 1) and HG of the
// rows' head vectors (every layer's K and V heads). Keeping a sequence's rows
// together lets the V heads be written well: V is stored channel-major inside
// 32-position blocks, so one channel's values at consecutive positions are
// adjacent in memory; each V head is staged in LDS and written transposed, 16
// lanes per channel run (a wave store covers 4 channels x 16 positions). The
// tile's (cos, sin) table is built once per workgroup. The kernel also
// advances ctx_len: it reads the rows' positions from a snapshot of ctx_len
// that the projection before it took, so one workgroup may update the live
// array at any time (one launch instead of a separate length update).
// ---------------------------------------------------------------------------
constexpr int kNrRows = 16;

__device__ __forceinline__ float2 rope_cs(const NormRopeArgs& p, int pos, int pair) {
  float c = 1.f, s = 0.f;
  if (p.rope_theta > 0.f) {
    constexpr double kTwoPiHi = 6.283185307179586;         // nearest double to 2 pi
    constexpr double kTwoPiLo = 2.4492935982947064e-16;    // 2 pi - kTwoPiHi
    const double ang = (double)pos * p.inv_freq[pair];
    const double k = rint(ang * (1.0 / kTwoPiHi));
    const double r = fma(-k, kTwoPiLo, fma(-k, kTwoPiHi, ang));
    sincosf((float)r, &s, &c);
  }
  return make_float2(c, s);
}

// Sum over the PAIRS lanes of one head (lanes with the same `sub`).
template <int PAIRS>
__device__ __forceinline__ float head_sum(float v) {
#pragma unroll
  for (int o = PAIRS / 2; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Per-head RMSNorm (gain g0, g1 of the lane's pair) and rotation of one pair.
template <int HD>
__device__ __forceinline__ void norm_rope_pair(float x0, float x1, float g0, float g1, float eps,
                                               float2 cs, float& o0, float& o1) {
  const float ss = head_sum<HD / 2>(x0 * x0 + x1 * x1);
  const float inv = rsqrtf(ss / (float)HD + eps);
  const float y0 = x0 * inv * g0, y1 = x1 * inv * g1;
  o0 = y0 * cs.x - y1 * cs.y;
  o1 = y1 * cs.x + y0 * cs.y;
}

// Rotary pairs of one row: a head vector of HD channels is HD/2 pairs
// (channel c with c + HD/2). A wave covers 64 / (HD/2) heads at once: lane
// (sub, c) with c = lane % (HD/2) owns pair c of the iteration's head sub.
// The rotation angle depends only on the position and the pair index, so
// each lane computes its (cos, sin) once per row for all the heads it takes.
// The angle pos * inv_freq is formed in double (positions reach tens of
// thousands of radians), reduced by 2 pi in double (Cody-Waite: 2 pi as the
// nearest double plus its remainder), and the reduced angle in [-pi, pi]
// goes to the fp32 sincos.
template <int HD>
struct RopeLane {
  static constexpr int PAIRS = HD / 2;
  static constexpr int HPW = 64 / PAIRS;  // heads per wave iteration
  float c = 1.f, s = 0.f;
  __device__ RopeLane(const NormRopeArgs& p, int pos, int pair) {
    if (p.rope_theta > 0.f) {
      constexpr double kTwoPiHi = 6.283185307179586;         // nearest double to 2 pi
      constexpr double kTwoPiLo = 2.4492935982947064e-16;    // 2 pi - kTwoPiHi
      const double ang = (double)pos * p.inv_freq[pair];
      const double k = rint(ang * (1.0 / kTwoPiHi));
      const double r = fma(-k, kTwoPiLo, fma(-k, kTwoPiHi, ang));
      sincosf((float)r, &s, &c);
    }
  }
};

// Heads (or append columns) per workgroup: 4 waves x IT iterations x
// RopeLane::HPW heads per iteration. A wave loads all its heads' pairs
// first, then normalises and stores them: one memory latency per wave. Few
// rows (batch 1) take IT = 1 for more waves in flight; many take IT = 4,
// which shares each row's rotary angles over more heads.
template <int HD, int IT>
__host__ __device__ constexpr int nr_heads_per_wg() { return 4 * IT * (64 / (HD / 2)); }

// V heads of the forward mode: the 16 workgroups of sequence s (slots
// s*16 .. s*16+15, last grid row) split its Hkv*HD value columns; each copies
// its columns of the block's rows through LDS (row-wise loads) and writes
// them to the channel-major cache blocks a column at a time, four threads per
// column, each with four consecutive positions (one 32-byte run per column
// instead of one 2-byte store per channel and position).
constexpr int kNrVCols = 128;  // columns a workgroup stages at a time
template <typename T, int HD>
__device__ __forceinline__ void nr_fwd_values(const NormRopeArgs& p, int s, int part) {
  __shared__ float tile[16][kNrVCols + 1];
  const int Hq = p.n_heads, Hkv = p.n_kv_heads;
  const int total = Hkv * HD, per = (total + 15) / 16;
  const int col_lo = part * per, col_hi = min(total, col_lo + per);
  int cl = p.ctx_len[s];
  cl = cl < 0 ? 0 : cl;
  const float* src = p.src + (int64_t)s * p.block * p.src_stride + (int64_t)(Hq + Hkv) * HD;
  for (int c0 = col_lo; c0 < col_hi; c0 += kNrVCols) {
    const int nc = min(kNrVCols, col_hi - c0);
    if (c0 > col_lo) __syncthreads();  // the previous chunk's reads are done
    // Every load of the chunk in flight at once (16 rows x 128 columns over
    // the 256 threads: up to 8 each), then into LDS.
    constexpr int kPer = 16 * kNrVCols / 256;
    float v[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int idx = threadIdx.x + 256 * u, r = idx / nc, cc = idx - r * nc;
      v[u] = idx < 16 * nc && r < p.block ? src[(int64_t)r * p.src_stride + c0 + cc] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int idx = threadIdx.x + 256 * u, r = idx / nc, cc = idx - r * nc;
      if (idx < 16 * nc) tile[r][cc] = v[u];
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < 4 * nc; idx += blockDim.x) {
      const int cc = idx >> 2, q = idx & 3, col = c0 + cc;
      const int g = col / HD, ch = col - g * HD;
      T* vb = reinterpret_cast<T*>(p.v_cache) + (size_t)(s * Hkv + g) * p.cap * HD;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * q + e, pos = cl + r;
        if (r < p.block && pos < p.cap)
          vb[(size_t)(pos / kKeyBlock) * HD * kKeyBlock + (size_t)ch * kKeyBlock + pos % kKeyBlock] =
              from_f32<T>(tile[r][cc]);
      }
    }
  }
}

// Forward mode: grid (batch * 16 block slots, Q/K head groups + 1); workgroup
// (slot, y) takes Q/K heads y * nr_heads_per_wg + (it * 4 + wave) * HPW + sub
// of the row's Hq + Hkv; the last grid row writes the V heads
// (nr_fwd_values). Slots i >= block only zero-fill the padded Q rows.
template <typename T, int HD, int IT>
__global__ __launch_bounds__(256) void norm_rope_fwd_kernel(NormRopeArgs p) {
  using RL = RopeLane<HD>;
  const int slot = blockIdx.x, s = slot / 16, i = slot % 16;
  if (blockIdx.y == gridDim.y - 1) {
    nr_fwd_values<T, HD>(p, s, i);
    return;
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int sub = lane / RL::PAIRS, c = lane % RL::PAIRS;
  const int Hq = p.n_heads, Hkv = p.n_kv_heads, NQK = Hq + Hkv;
  const int hbase = blockIdx.y * nr_heads_per_wg<HD, IT>() + wave * RL::HPW + sub;
  if (i >= p.block) {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int h = hbase + it * 4 * RL::HPW;
      if (h < Hq) {
        T* qo = reinterpret_cast<T*>(p.q_out) + (((size_t)s * Hq + h) * 16 + i) * HD;
        qo[c] = from_f32<T>(0.f);
        qo[c + RL::PAIRS] = from_f32<T>(0.f);
      }
    }
    return;
  }
  const int m = s * p.block + i;
  const float* src = p.src + (int64_t)m * p.src_stride;
  float x0[IT], x1[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int hc = min(hbase + it * 4 * RL::HPW, NQK - 1);
    x0[it] = src[hc * HD + c];
    x1[it] = src[hc * HD + c + RL::PAIRS];
  }
  int cl = p.ctx_len[s];
  cl = cl < 0 ? 0 : cl;
  const int pos = cl + i;
  const bool in_cap = pos < p.cap;
  if (!in_cap && threadIdx.x == 0 && blockIdx.y == 0 && p.dev_status)
    atomicOr(p.dev_status, DFLASH_DEV_CAPACITY);
  const RL rope(p, pos, c);
  const T* qg = reinterpret_cast<const T*>(p.q_norm[0]);
  const T* kg = reinterpret_cast<const T*>(p.k_norm[0]);
  const float qg0 = to_f32(qg[c]), qg1 = to_f32(qg[c + RL::PAIRS]);
  const float kg0 = to_f32(kg[c]), kg1 = to_f32(kg[c + RL::PAIRS]);
  // Every lane of an iteration takes part (the head sums shuffle across it);
  // heads past the last were clamped and are not stored.
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int h = hbase + it * 4 * RL::HPW;
    const int hc = min(h, NQK - 1);
    const bool is_q = hc < Hq;
    float o0, o1;
    norm_rope_pair<HD>(x0[it], x1[it], is_q ? qg0 : kg0, is_q ? qg1 : kg1, p.eps,
                       make_float2(rope.c, rope.s), o0, o1);
    if (h >= NQK) continue;
    if (is_q) {
      T* qo = reinterpret_cast<T*>(p.q_out) + (((size_t)s * Hq + h) * 16 + i) * HD;
      qo[c] = from_f32<T>(o0);
      qo[c + RL::PAIRS] = from_f32<T>(o1);
    } else if (in_cap) {
      const int g = h - Hq;
      T* kr = reinterpret_cast<T*>(p.k_cache) + ((size_t)(s * Hkv + g) * p.cap + pos) * HD;
      kr[c] = from_f32<T>(o0);
      kr[c + RL::PAIRS] = from_f32<T>(o1);
    }
  }
}

struct NrTile {
  int s;       // sequence (-1: this workgroup has no tile)
  int row0;    // first source row
  int nrows;   // rows in the tile (<= 16)
  int pos0;    // cache position of the first row
};

// Where the tile of workgroup blockIdx.x lies (p.ctx_len is the snapshot).
//   Accepted rows: sequence blockIdx.x, rows s*B + i for i <= accept_len[s],
//     at ctx_len[s] + i.
//   Prefix offsets: the sequences' new rows cut into tiles of 16
//     (ceil(n_s / 16) tiles for sequence s, in order); wave 0 scans the tile
//     counts 64 sequences at a time. Rows outside [0, n_tok) are never read.
__device__ __forceinline__ NrTile nr_locate(const NormRopeArgs& p, int* sh) {
  NrTile t{-1, 0, 0, 0};
  if (p.accept_len) {
    const int s = blockIdx.x;
    if (s >= p.batch) return t;
    int cl = p.ctx_len[s];
    cl = cl < 0 ? 0 : cl;
    t.s = s;
    t.row0 = s * p.block;
    t.nrows = accepted_rows(p.accept_len[s], p.block);
    t.pos0 = cl;
    return t;
  }
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x, T = blockIdx.x;
    int carry = 0, found = -1, before = 0;
    for (int base = 0; base < p.batch && found < 0; base += 64) {
      const int s = base + lane;
      int n = 0;
      if (s < p.batch) n = max(0, p.cu_new[s + 1] - p.cu_new[s]);
      const int own = (n + kNrRows - 1) / kNrRows;
      int v = own;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(v, o);
        if (lane >= o) v += u;
      }
      // first lane whose inclusive prefix passes T
      const unsigned long long hit = __ballot(s < p.batch && carry + v > T);
      if (hit) {
        const int l = __ffsll((long long)hit) - 1;
        found = base + l;
        before = carry + __shfl(v - own, l);
      }
      carry += __shfl(v, 63);
    }
    if (lane == 0) {
      sh[0] = found;
      sh[1] = found < 0 ? 0 : T - before;
    }
  }
  __syncthreads();
  const int s = sh[0];
  if (s < 0) return t;
  const int ti = sh[1];
  const int n = max(0, p.cu_new[s + 1] - p.cu_new[s]);
  int cl = p.ctx_len[s];
  cl = cl < 0 ? 0 : cl;
  t.s = s;
  t.row0 = p.cu_new[s] + kNrRows * ti;
  t.nrows = min(kNrRows, n - kNrRows * ti);
  if (t.row0 < 0) t.nrows = 0;
  t.nrows = min(t.nrows, p.n_tok - t.row0);
  t.pos0 = cl + kNrRows * ti;
  return t;
}

// Append only, workgroup (0, 0): ctx_len[s] = snapshot[s] + rows of s (the
// kernel reads positions from the snapshot, so this may happen at any time),
// clamped to the capacity, with the offset checks of the prefix mode.
__device__ __forceinline__ void nr_update_lengths(const NormRopeArgs& p) {
  if (threadIdx.x == 0 && !p.accept_len &&
      (p.cu_new[0] != 0 || p.cu_new[p.batch] != p.n_tok) && p.dev_status)
    atomicOr(p.dev_status, DFLASH_DEV_OFFSETS);
  for (int s = threadIdx.x; s < p.batch; s += blockDim.x) {
    int n;
    if (p.accept_len) {
      const int a = p.accept_len[s];
      if ((a < 0 || a >= p.block) && p.dev_status) atomicOr(p.dev_status, DFLASH_DEV_OFFSETS);
      n = accepted_rows(a, p.block);
    } else {
      n = p.cu_new[s + 1] - p.cu_new[s];
      if (n < 0) {
        if (p.dev_status) atomicOr(p.dev_status, DFLASH_DEV_OFFSETS);
        n = 0;
      }
    }
    int cl = p.ctx_len[s];
    cl = cl < 0 ? 0 : cl;
    int nl = cl + n;
    if (nl > p.cap) {
      if (p.dev_status) atomicOr(p.dev_status, DFLASH_DEV_CAPACITY);
      nl = p.cap;
    }
    p.ctx_len_out[s] = nl;
  }
}

// grid (tiles, head groups of HG). Head h = l * 2 Hkv + hh of the stacked
// context projection's row: hh < Hkv a key head of layer l, else a value head.
template <typename T, int HD, int HG>
__global__ __launch_bounds__(256) void norm_rope_append_kernel(NormRopeArgs p) {
  constexpr int PAIRS = HD / 2;
  constexpr int HPW = 64 / PAIRS;                    // items per wave step
  constexpr int NIT = kNrRows * HG / (4 * HPW);      // items per lane group
  constexpr int VS = HD + 4;                         // LDS row stride of a staged V head
  static_assert(NIT * 4 * HPW == kNrRows * HG, "items split evenly");
  __shared__ float2 rtab[kNrRows * PAIRS];
  __shared__ float vst[HG][kNrRows][VS];
  __shared__ int sh[2];

  if (blockIdx.x == 0 && blockIdx.y == 0) nr_update_lengths(p);
  const NrTile tile = nr_locate(p, sh);
  if (tile.s < 0 || tile.nrows <= 0) return;
  const int s = tile.s;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int sub = lane / PAIRS, c = lane % PAIRS;
  const int Hkv = p.n_kv_heads;
  const int NH = p.n_layers * 2 * Hkv;
  const int h0 = blockIdx.y * HG;
  // Rows at or past the capacity are dropped (and flagged).
  const int nvalid = max(0, min(tile.nrows, p.cap - tile.pos0));
  if (nvalid < tile.nrows && threadIdx.x == 0 && blockIdx.y == 0 && p.dev_status)
    atomicOr(p.dev_status, DFLASH_DEV_CAPACITY);

  for (int e = threadIdx.x; e < kNrRows * PAIRS; e += blockDim.x)
    rtab[e] = (e / PAIRS) < tile.nrows ? rope_cs(p, tile.pos0 + e / PAIRS, e % PAIRS)
                                       : make_float2(1.f, 0.f);

  // Phase 1: every (head, row) item of the lane group (lane (sub, c) owns
  // pair c of item sub): loads first, then norm + rotation; K rows are stored
  // directly, V rows staged in LDS.
  float x0[NIT], x1[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int item = (it * 4 + wave) * HPW + sub;
    const int k = item / kNrRows, i = item % kNrRows, h = h0 + k;
    x0[it] = x1[it] = 0.f;
    if (h < NH && i < tile.nrows) {
      const float* src = p.src + (int64_t)(tile.row0 + i) * p.src_stride + (int64_t)h * HD;
      x0[it] = src[c];
      x1[it] = src[c + PAIRS];
    }
  }
  // The projection's K-slice partials, added in slice order (one batch of
  // loads per slice).
  for (int z = 1; z < p.src_slices; ++z) {
    float y0[NIT], y1[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int item = (it * 4 + wave) * HPW + sub;
      const int k = item / kNrRows, i = item % kNrRows, h = h0 + k;
      y0[it] = y1[it] = 0.f;
      if (h < NH && i < tile.nrows) {
        const float* src = p.src + z * p.slice_stride + (int64_t)(tile.row0 + i) * p.src_stride +
                           (int64_t)h * HD;
        y0[it] = src[c];
        y1[it] = src[c + PAIRS];
      }
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      x0[it] += y0[it];
      x1[it] += y1[it];
    }
  }
  __syncthreads();  // rtab
  const size_t layer_stride = (size_t)p.cache_batch * Hkv * p.cap * HD;
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int item = (it * 4 + wave) * HPW + sub;
    const int k = item / kNrRows, i = item % kNrRows, h = h0 + k;
    const int l = min(h, NH - 1) / (2 * Hkv), hh = min(h, NH - 1) % (2 * Hkv);
    if (hh >= Hkv) {  // value head (or past the last head): staged
      vst[k][i][c] = x0[it];
      vst[k][i][c + PAIRS] = x1[it];
      continue;
    }
    const int g = hh;
    const T* gp = reinterpret_cast<const T*>(p.k_norm[l]);
    float o0, o1;
    norm_rope_pair<HD>(x0[it], x1[it], to_f32(gp[c]), to_f32(gp[c + PAIRS]), p.eps,
                       rtab[i * PAIRS + c], o0, o1);
    if (h < NH && i < nvalid) {
      T* kr = reinterpret_cast<T*>(p.k_cache) + l * layer_stride +
              ((size_t)(s * Hkv + g) * p.cap + tile.pos0 + i) * HD;
      kr[c] = from_f32<T>(o0);
      kr[c + PAIRS] = from_f32<T>(o1);
    }
  }
  __syncthreads();  // vst

  // Phase 2: the staged V heads, transposed: thread (c4, j) writes channel
  // 16 cg + c4 at position pos0 + j, cg = 0 .. HD/16 - 1.
  const int j = threadIdx.x & 15, c4 = threadIdx.x >> 4;
  const int pos = tile.pos0 + j;
#pragma unroll
  for (int k = 0; k < HG; ++k) {
    const int h = h0 + k;
    if (h >= NH) break;
    const int l = h / (2 * Hkv), hh = h % (2 * Hkv);
    if (hh < Hkv || j >= nvalid) continue;
    const int g = hh - Hkv;
    T* vb = reinterpret_cast<T*>(p.v_cache) + l * layer_stride + (size_t)(s * Hkv + g) * p.cap * HD +
            (size_t)(pos / kKeyBlock) * HD * kKeyBlock + (pos % kKeyBlock);
#pragma unroll
    for (int cg = 0; cg < HD / 16; ++cg) {
      const int ch = 16 * cg + c4;
      vb[(size_t)ch * kKeyBlock] = from_f32<T>(vst[k][j][ch]);
    }
  }
}

// Grid: rows x (Q/K head groups + one row for the V heads).
template <int IT>
static hipError_t launch_nr_it(int dtype, const NormRopeArgs& a, int rows, int n_cols,
                               hipStream_t st) {
  const bool bf = dtype == DFLASH_BF16;
  const dim3 blk(256);
#define DF_NR(K, T, HD)                                                                     \
  hipLaunchKernelGGL((K<T, HD, IT>), dim3(rows, (n_cols + nr_heads_per_wg<HD, IT>() - 1) / \
                                                   nr_heads_per_wg<HD, IT>() + 1),          \
                     blk, 0, st, a)
  if (a.head_dim == 128) {
    if (bf) DF_NR(norm_rope_fwd_kernel, bf16, 128);
    else DF_NR(norm_rope_fwd_kernel, float, 128);
  } else if (a.head_dim == 64) {
    if (bf) DF_NR(norm_rope_fwd_kernel, bf16, 64);
    else DF_NR(norm_rope_fwd_kernel, float, 64);
  } else {
    return hipErrorInvalidValue;
  }
#undef DF_NR
  return hipGetLastError();
}

// rows x n_cols head vectors; IT = 1 below 128 rows.
static hipError_t launch_nr_fwd(int dtype, const NormRopeArgs& a, int rows, int n_cols,
                                hipStream_t st) {
  if (rows < 128) return launch_nr_it<1>(dtype, a, rows, n_cols, st);
  return launch_nr_it<4>(dtype, a, rows, n_cols, st);
}

template <int HG>
static hipError_t launch_nr_append(int dtype, const NormRopeArgs& a, int tiles, int n_heads,
                                   hipStream_t st) {
  const dim3 grid(tiles, (n_heads + HG - 1) / HG), blk(256);
  const bool bf = dtype == DFLASH_BF16;
  if (a.head_dim == 128) {
    if (bf) hipLaunchKernelGGL((norm_rope_append_kernel<bf16, 128, HG>), grid, blk, 0, st, a);
    else hipLaunchKernelGGL((norm_rope_append_kernel<float, 128, HG>), grid, blk, 0, st, a);
  } else if (a.head_dim == 64) {
    if (bf) hipLaunchKernelGGL((norm_rope_append_kernel<bf16, 64, HG>), grid, blk, 0, st, a);
    else hipLaunchKernelGGL((norm_rope_append_kernel<float, 64, HG>), grid, blk, 0, st, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// The rotary inverse frequencies of the config, in double.
static NormRopeArgs with_inv_freq(const NormRopeArgs& a0) {
  NormRopeArgs a = a0;
  for (int i = 0; i < 64; ++i)
    a.inv_freq[i] = (a.rope_theta > 0.f && 2 * i < a.head_dim)
                        ? std::pow((double)a.rope_theta, -2.0 * i / (double)a.head_dim)
                        : 0.0;
  return a;
}

hipError_t launch_norm_rope_forward(int dtype, const NormRopeArgs& a, hipStream_t st) {
  return launch_nr_fwd(dtype, with_inv_freq(a), a.batch * 16, a.n_heads + a.n_kv_heads, st);
}

// Heads per workgroup: 2 while the tiles are few (more workgroups in
// flight), 4 from 64 tiles (each row's rotary table serves more heads).

hipError_t launch_norm_rope_append(int dtype, const NormRopeArgs& a, hipStream_t st) {
  if (a.n_tok <= 0 || !a.ctx_len_out) return hipErrorInvalidValue;
  if (a.block > kNrRows) return hipErrorInvalidValue;
  // prefix offsets: at most ceil(n_tok / 16) + batch tiles (each sequence's
  // last tile may be partial)
  const int tiles = a.accept_len ? a.batch : (a.n_tok + kNrRows - 1) / kNrRows + a.batch;
  const int nh = a.n_layers * 2 * a.n_kv_heads;
  if (tiles < 64) return launch_nr_append<2>(dtype, with_inv_freq(a), tiles, nh, st);
  return launch_nr_append<4>(dtype, with_inv_freq(a), tiles, nh, st);
}

// One workgroup per draft row: its 1024 threads reduce the row's per-column
// (max, argmax) keys from the LM head (thousands of columns at batch 1) into
// the draft token. With targets, the last row of a sequence to finish (a
// per-sequence arrival counter, zeroed by the embedding kernel at the start
// of the forward) applies the greedy accept rule to the sequence's drafts.
__global__ __launch_bounds__(1024) void argmax_rows_kernel(const unsigned long long* amax,
                                                           int64_t stride, int n_cols, int block,
                                                           int32_t* drafts, const int32_t* targets,
                                                           int32_t* accept_len, int32_t* bonus,
                                                           int32_t* arrivals) {
  __shared__ unsigned long long red[16];
  __shared__ int is_last;
  const int row = blockIdx.x, m = block - 1, s = row / m;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const unsigned long long* keys = amax + (int64_t)row * stride;
  unsigned long long best = 0ull;
#pragma unroll 4
  for (int c = threadIdx.x; c < n_cols; c += 1024) {
    const unsigned long long k = keys[c];
    best = k > best ? k : best;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned long long other = __shfl_xor(best, o);
    best = other > best ? other : best;
  }
  if (lane == 0) red[wave] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 16; ++w) best = red[w] > best ? red[w] : best;
    best = red[0] > best ? red[0] : best;
    drafts[row] = (int32_t)argmax_index(best);
    is_last = 0;
    if (targets) {
      __threadfence();  // the draft is visible before the arrival is counted
      is_last = atomicAdd(&arrivals[s], 1) == m - 1;
    }
  }
  __syncthreads();
  if (is_last && threadIdx.x == 0) {
    __threadfence();  // see every row's draft
    const volatile int32_t* d = drafts + (int64_t)s * m;
    const int32_t* t = targets + (int64_t)s * block;
    int a = 0;
    while (a < m && d[a] == t[a]) ++a;
    accept_len[s] = a;
    bonus[s] = t[a];
    arrivals[s] = 0;
  }
}

// The same for a sequence's rows together: one workgroup per sequence, wave
// w reduces row s*m + w (m <= 16), and the workgroup applies the accept rule
// to the drafts it just computed (no cross-workgroup handoff). For rows of
// few keys (the MFMA LM head's column blocks); rows of thousands of keys
// (the weight-streaming LM head's tiles) keep a workgroup each.
__global__ __launch_bounds__(1024) void argmax_seq_kernel(const unsigned long long* amax,
                                                          int64_t stride, int n_cols, int block,
                                                          int32_t* drafts, const int32_t* targets,
                                                          int32_t* accept_len, int32_t* bonus) {
  __shared__ int32_t tok[16];
  const int s = blockIdx.x, m = block - 1;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (wave < m) {
    const int64_t row = (int64_t)s * m + wave;
    const unsigned long long* keys = amax + row * stride;
    unsigned long long best = 0ull;
#pragma unroll 4
    for (int c = lane; c < n_cols; c += 64) {
      const unsigned long long k = keys[c];
      best = k > best ? k : best;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const unsigned long long other = __shfl_xor(best, o);
      best = other > best ? other : best;
    }
    if (lane == 0) {
      const int32_t t = (int32_t)argmax_index(best);
      drafts[row] = t;
      tok[wave] = t;
    }
  }
  __syncthreads();
  if (targets && threadIdx.x == 0) {
    const int32_t* t = targets + (int64_t)s * block;
    int a = 0;
    while (a < m && tok[a] == t[a]) ++a;
    accept_len[s] = a;
    bonus[s] = t[a];
  }
}

hipError_t launch_argmax_accept(const unsigned long long* amax, int64_t stride, int n_cols,
                                int batch, int block, int32_t* drafts, const int32_t* targets,
                                int32_t* accept_len, int32_t* bonus, int32_t* arrivals,
                                hipStream_t st) {
  if (batch <= 0 || block < 2 || block > 17) return block == 1 ? hipSuccess : hipErrorInvalidValue;
  if (targets && !arrivals) return hipErrorInvalidValue;
  if (n_cols <= 2048) {
    hipLaunchKernelGGL(argmax_seq_kernel, dim3(batch), dim3(1024), 0, st, amax, stride, n_cols,
                       block, drafts, targets, accept_len, bonus);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(argmax_rows_kernel, dim3(batch * (block - 1)), dim3(1024), 0, st, amax, stride,
                     n_cols, block, drafts, targets, accept_len, bonus, arrivals);
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

__global__ void ctx_len_add_kernel(int32_t* ctx_len, const int32_t* cu_new,
                                   const int32_t* accept_len, int block, int batch, int n_tok,
                                   int cap, int32_t* dev_status) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (!accept_len && s == 0 && (cu_new[0] != 0 || cu_new[batch] != n_tok) && dev_status)
    atomicOr(dev_status, DFLASH_DEV_OFFSETS);
  if (s >= batch) return;
  int n;
  if (accept_len) {
    const int a = accept_len[s];
    if ((a < 0 || a >= block) && dev_status) atomicOr(dev_status, DFLASH_DEV_OFFSETS);
    n = accepted_rows(a, block);
  } else {
    n = cu_new[s + 1] - cu_new[s];
    if (n < 0) {
      if (dev_status) atomicOr(dev_status, DFLASH_DEV_OFFSETS);
      n = 0;
    }
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

hipError_t launch_ctx_len_add(int32_t* ctx_len, const int32_t* cu_new, const int32_t* accept_len,
                              int block, int batch, int n_tok, int cap, int32_t* dev_status,
                              hipStream_t st) {
  hipLaunchKernelGGL(ctx_len_add_kernel, dim3((batch + 63) / 64), dim3(64), 0, st, ctx_len, cu_new,
                     accept_len, block, batch, n_tok, cap, dev_status);
  return hipGetLastError();
}

}  // namespace dflash
