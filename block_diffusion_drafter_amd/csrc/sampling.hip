// Temperature > 0: drafting by sampling and speculative verification with
// residual resampling ("DFlash: Why a Diffusion Drafter Can Accelerate an
// Autoregressive Model", sec. 4.2, eqs. 6-8 and Algorithm 1).
//
// Random numbers: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC 2011). Element i of (row, round, stream)
// is word i % 4 of the block at counter (i / 4, row, round, stream) under key
// (low, high half of the 64-bit seed); a uniform is ((w >> 9) + 0.5) * 2^-23
// (24 significant bits: exact in fp32, never 0 or 1). A categorical draw is a
// Gumbel-max: the argmax of log-probability + (-log(-log u)) over the
// support, lowest index on ties.
//
// Every reduction over the vocabulary is split over workgroups of 8192
// logits: a thread loads its 32 logits (8 steps of 4 consecutive ones) before
// using any, takes their max and then their sum of exponentials (one exp per
// logit, no data-dependent branch), and draws one Philox block per 4 logits;
// small kernels merge the splits.
#include <cmath>
#include <mutex>

#include "common.h"
#include "internal.h"

namespace dflash {

namespace {

constexpr int kSplit = 8192;  // logits per workgroup
constexpr int kThreads = 256;

constexpr int kIt = kSplit / (4 * kThreads);  // 4-logit steps per thread and split

// Ten rounds: words 0 and 2 times the two multipliers (32 x 32 -> 64-bit
// products), the products' halves exchanged with words 1 and 3 xor the round
// key, the key bumped by the two Weyl constants between rounds.
__device__ __forceinline__ void philox4x32(uint32_t c[4], uint32_t k0, uint32_t k1) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)M0 * c[0];
    const uint64_t p1 = (uint64_t)M1 * c[2];
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = (uint32_t)p1;
    c[2] = n2;
    c[3] = (uint32_t)p0;
    k0 += W0;
    k1 += W1;
  }
}

// The four uniforms of elements 4q .. 4q+3 of (row, round, stream).
__device__ __forceinline__ void uniforms4(uint64_t seed, uint32_t q, uint32_t row, uint32_t rnd,
                                          uint32_t stream, float u[4]) {
  uint32_t c[4] = {q, row, rnd, stream};
  philox4x32(c, (uint32_t)seed, (uint32_t)(seed >> 32));
#pragma unroll
  for (int w = 0; w < 4; ++w) u[w] = ((float)(c[w] >> 9) + 0.5f) * 0x1p-23f;
}

// This thread's logits of a split of IT*4*kThreads logits: step i holds
// elements v0 + 4*kThreads*i .. +3 (v0 = split*IT*4*kThreads +
// 4*threadIdx.x), -inf past V; every load is issued before any value is used.
template <int IT = kIt>
__device__ __forceinline__ void load_split(const float* l, int V, int split, float x[IT][4]) {
  const int v0 = split * (IT * 4 * kThreads) + 4 * (int)threadIdx.x;
  if ((V & 3) == 0 && (reinterpret_cast<uintptr_t>(l) & 15) == 0) {
    // whole 16-byte groups: v < V implies v + 3 < V
    const float4* l4 = reinterpret_cast<const float4*>(l);
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int v = v0 + 4 * kThreads * i;
      float4 t = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      if (v < V) t = l4[v >> 2];
      x[i][0] = t.x;
      x[i][1] = t.y;
      x[i][2] = t.z;
      x[i][3] = t.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < IT; ++i)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int v = v0 + 4 * kThreads * i + w;
        x[i][w] = v < V ? l[v] : -INFINITY;
      }
  }
}

// -log(-log u) from two hardware base-2 logarithms (v_log_f32, relative
// error about 1 ulp; u in [2^-24, 1 - 2^-24] and a = -log2 u in
// [8.6e-8, 24] are normal numbers, so no denormal scaling is needed):
// -log(-log u) = -log(a ln 2) = -log(ln 2) - ln 2 * log2 a.
__device__ __forceinline__ float gumbel(float u) {
  const float a = -__builtin_amdgcn_logf(u);
  return fmaf(-0.693147180559945309f, __builtin_amdgcn_logf(a), 0.366512920581664327f);
}

// Order-preserving key of (score, index): larger score wins, lower index on ties.
__device__ __forceinline__ unsigned long long okey(float v, unsigned idx) {
  return argmax_key(v, idx);
}

// Online log-sum-exp state (max, sum of exp(x - max)).
struct Lse {
  float m = -INFINITY, s = 0.f;
  __device__ void add(float x) {
    if (x > m) {
      s = s * __expf(m - x) + 1.f;
      m = x;
    } else {
      s += __expf(x - m);
    }
  }
  __device__ void merge(float m2, float s2) {
    if (m2 == -INFINITY) return;
    if (m2 > m) {
      s = s * __expf(m - m2) + s2;
      m = m2;
    } else {
      s += s2 * __expf(m2 - m);
    }
  }
  __device__ float value() const { return m + logf(s); }
};

// Log-sum-exp state of a thread's scaled logits (scaled in place): the max
// first, then the sum of exp(x - max).
__device__ __forceinline__ Lse tile_lse(float x[kIt][4], float inv_t) {
  Lse l;
#pragma unroll
  for (int i = 0; i < kIt; ++i)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      x[i][w] *= inv_t;
      l.m = fmaxf(l.m, x[i][w]);
    }
  if (l.m != -INFINITY) {
#pragma unroll
    for (int i = 0; i < kIt; ++i)
#pragma unroll
      for (int w = 0; w < 4; ++w) l.s += __expf(x[i][w] - l.m);
  }
  return l;
}

__device__ __forceinline__ unsigned long long block_max_key(unsigned long long k,
                                                            unsigned long long* sh) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned long long x = __shfl_xor(k, o);
    k = x > k ? x : k;
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sh[w] = k;
  __syncthreads();
  unsigned long long r = 0ull;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) r = sh[i] > r ? sh[i] : r;
  __syncthreads();
  return r;
}

__device__ __forceinline__ void block_lse(Lse& l, float* shm, float* shs) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) l.merge(__shfl_xor(l.m, o), __shfl_xor(l.s, o));
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    shm[w] = l.m;
    shs[w] = l.s;
  }
  __syncthreads();
  Lse r;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) r.merge(shm[i], shs[i]);
  __syncthreads();
  l = r;
}

struct SplitStat {        // per (row, split)
  unsigned long long key;  // Gumbel-max key (sampling) or unused
  float m, s;              // log-sum-exp partial of logits / T
};

// ---- drafting -----------------------------------------------------------

__global__ __launch_bounds__(kThreads) void sample_split_kernel(const float* logits, int64_t ld,
                                                                 int V, float inv_t, uint64_t seed,
                                                                 int rnd, SplitStat* part,
                                                                 int nsplit) {
  __shared__ unsigned long long shk[kThreads / 64];
  __shared__ float shm[kThreads / 64], shs[kThreads / 64];
  const int split = blockIdx.x, row = blockIdx.y;
  const float* l = logits + (int64_t)row * ld;
  float x[kIt][4];
  load_split(l, V, split, x);
  Lse lse = tile_lse(x, inv_t);
  // The thread's best perturbed score: it visits its indices in increasing
  // order and keeps the first of equal scores, the lowest index on ties.
  const int v0 = split * kSplit + 4 * (int)threadIdx.x;
  float best = -INFINITY;
  int best_v = v0;
  auto step = [&](int i, bool full) {
    const int v = v0 + 4 * kThreads * i;
    if (!full && v >= V) return;
    float u[4];
    uniforms4(seed, (uint32_t)(v >> 2), (uint32_t)row, (uint32_t)rnd, 0u, u);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float sc = x[i][w] + gumbel(u[w]);
      if ((full || v + w < V) && sc > best) {
        best = sc;
        best_v = v + w;
      }
    }
  };
  if ((split + 1) * kSplit <= V) {
#pragma unroll
    for (int i = 0; i < kIt; ++i) step(i, true);
  } else {
#pragma unroll
    for (int i = 0; i < kIt; ++i) step(i, false);
  }
  unsigned long long key = v0 < V ? okey(best, (unsigned)best_v) : 0ull;
  key = block_max_key(key, shk);
  block_lse(lse, shm, shs);
  if (threadIdx.x == 0) part[(int64_t)row * nsplit + split] = SplitStat{key, lse.m, lse.s};
}

__global__ void sample_finish_kernel(const float* logits, int64_t ld, float inv_t,
                                     const SplitStat* part, int nsplit, int rows, int32_t* tokens,
                                     float* logq) {
  const int row = blockIdx.x * blockDim.x + threadIdx.x;
  if (row >= rows) return;
  unsigned long long key = 0ull;
  Lse lse;
  // Splits in groups of 8, every load of a group before its merges (in
  // split order).
  for (int i0 = 0; i0 < nsplit; i0 += 8) {
    SplitStat q[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      q[u] = i0 + u < nsplit ? part[(int64_t)row * nsplit + i0 + u] : SplitStat{0ull, -INFINITY, 0.f};
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      key = q[u].key > key ? q[u].key : key;
      lse.merge(q[u].m, q[u].s);
    }
  }
  const int tok = (int)argmax_index(key);
  tokens[row] = tok;
  if (logq) logq[row] = logits[(int64_t)row * ld + tok] * inv_t - lse.value();
}

// ---- verification -------------------------------------------------------

// Log-sum-exp partials of every target row (b x B) and draft row (b x m),
// draft rows stored after the target rows.
__global__ __launch_bounds__(kThreads) void verify_stats_kernel(const float* draft_logits,
                                                                 const float* target_logits,
                                                                 int batch, int B, int V,
                                                                 float inv_t, SplitStat* part,
                                                                 int nsplit) {
  __shared__ float shm[kThreads / 64], shs[kThreads / 64];
  const int split = blockIdx.x, r = blockIdx.y;  // r < batch*B: target; else draft
  const float* l = r < batch * B ? target_logits + (int64_t)r * V
                                 : draft_logits + (int64_t)(r - batch * B) * V;
  float x[kIt][4];
  load_split(l, V, split, x);
  Lse lse = tile_lse(x, inv_t);
  block_lse(lse, shm, shs);
  if (threadIdx.x == 0) part[(int64_t)r * nsplit + split] = SplitStat{0ull, lse.m, lse.s};
}

// Log-sum-exp of one row's logits / T from its split partials, merged in
// split order.
__device__ __forceinline__ float row_lse(const SplitStat* part, int64_t row, int nsplit) {
  Lse l;
  for (int i0 = 0; i0 < nsplit; i0 += 8) {  // groups of 8: loads first
    float m[8], sm[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const bool ok = i0 + u < nsplit;
      m[u] = ok ? part[row * nsplit + i0 + u].m : -INFINITY;
      sm[u] = ok ? part[row * nsplit + i0 + u].s : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) l.merge(m[u], sm[u]);
  }
  return l.value();
}

// Per sequence and split: the normalisers of the sequence's rows from the
// split partials (target rows; draft rows too unless log q of the drawn
// candidates is given, which recovers them as logit / T - log q), the accept
// test of every position (eq. 6, one thread per position) and the
// left-to-right scan for the first rejection, repeated by every split of the
// sequence (identical inputs, identical result); then the Gumbel-max partial
// over this split of the emitted law: the residual [p - q]_+ at the first
// rejected position (eq. 7), with the target law as fallback when the
// residual support is empty, or the target's next law when every candidate
// survived (bonus).
template <int IT>
__global__ __launch_bounds__(kThreads) void verify_residual_kernel(
    const int32_t* drafts, const float* draft_logits, const float* draft_logq,
    const float* target_logits, int batch, int B, int V, float inv_t, uint64_t seed, int rnd,
    const SplitStat* stats, int nsplit, unsigned long long* keys, int32_t* accept_out) {
  // nsplit: splits of the statistics (kSplit logits each); this kernel's own
  // splits over the emitted row are IT*4*kThreads logits each (gridDim.x).
  __shared__ unsigned long long shk[kThreads / 64];
  __shared__ int sh_ok[64];
  __shared__ float sh_lsep[64], sh_lseq[64];
  __shared__ int sh_a;
  const int split = blockIdx.x, s = blockIdx.y;
  const int m = B - 1;  // m + 1 <= 17 < kThreads
  if ((int)threadIdx.x <= m) {
    const int i = threadIdx.x;
    const float lse_p = row_lse(stats, (int64_t)s * B + i, nsplit);
    sh_lsep[i] = lse_p;
    if (i < m) {
      float u4[4];
      uniforms4(seed, (uint32_t)(i >> 2), (uint32_t)s, (uint32_t)rnd, 1u, u4);
      int y = drafts[(int64_t)s * m + i];
      y = y < 0 ? 0 : (y >= V ? V - 1 : y);  // ids outside the vocabulary are clamped
      const float xq = draft_logits[((int64_t)s * m + i) * V + y] * inv_t;
      float lq, lse_q;
      if (draft_logq) {
        lq = draft_logq[(int64_t)s * m + i];
        lse_q = xq - lq;
      } else {
        lse_q = row_lse(stats, (int64_t)batch * B + (int64_t)s * m + i, nsplit);
        lq = xq - lse_q;
      }
      sh_lseq[i] = lse_q;
      const float lp = target_logits[((int64_t)s * B + i) * V + y] * inv_t - lse_p;
      const float alpha = fminf(1.f, expf(lp - lq));
      sh_ok[i] = u4[i & 3] < alpha;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int a = 0;
    while (a < m && sh_ok[a]) ++a;
    sh_a = a;
    if (split == 0) accept_out[s] = a;
  }
  __syncthreads();
  const int a = sh_a;
  const float lse_p = sh_lsep[a];
  const float lse_q = a < m ? sh_lseq[a] : 0.f;
  const float* lp_row = target_logits + ((int64_t)s * B + a) * V;
  const float* lq_row = a < m ? draft_logits + ((int64_t)s * m + a) * V : nullptr;
  const uint32_t grow = (uint32_t)(s * B + a);
  float xp[IT][4], xq[IT][4];
  load_split<IT>(lp_row, V, split, xp);
  if (lq_row) load_split<IT>(lq_row, V, split, xq);
  unsigned long long kres = 0ull, kfb = 0ull;
  const int v0 = split * (IT * 4 * kThreads) + 4 * (int)threadIdx.x;
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int v = v0 + 4 * kThreads * i;
    if (v >= V) break;
    float u[4];
    uniforms4(seed, (uint32_t)(v >> 2), grow, (uint32_t)rnd, 2u, u);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int vv = v + w;
      if (vv >= V) continue;
      const float g = gumbel(u[w]);
      const float lp = xp[i][w] * inv_t - lse_p;
      const unsigned long long kf = okey(lp + g, (unsigned)vv);
      kfb = kf > kfb ? kf : kfb;
      if (lq_row) {
        const float d = expf(lp) - expf(xq[i][w] * inv_t - lse_q);
        if (d > 0.f) {
          const unsigned long long kr = okey(logf(d) + g, (unsigned)vv);
          kres = kr > kres ? kr : kres;
        }
      }
    }
  }
  kres = block_max_key(kres, shk);
  kfb = block_max_key(kfb, shk);
  if (threadIdx.x == 0) {
    keys[((int64_t)s * gridDim.x + split) * 2 + 0] = kres;
    keys[((int64_t)s * gridDim.x + split) * 2 + 1] = kfb;
  }
}

__global__ void verify_finish_kernel(const unsigned long long* keys, int nsplit, int batch, int B,
                                     const int32_t* accept_in, int32_t* accept_len,
                                     int32_t* out_token, int32_t* anchor_out) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= batch) return;
  unsigned long long kr = 0ull, kf = 0ull;
  for (int i0 = 0; i0 < nsplit; i0 += 8) {  // groups of 8: loads first
    unsigned long long a[8], b[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const bool ok = i0 + u < nsplit;
      a[u] = ok ? keys[((int64_t)s * nsplit + i0 + u) * 2 + 0] : 0ull;
      b[u] = ok ? keys[((int64_t)s * nsplit + i0 + u) * 2 + 1] : 0ull;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      kr = a[u] > kr ? a[u] : kr;
      kf = b[u] > kf ? b[u] : kf;
    }
  }
  const int a = accept_in[s];
  // residual draw when the rejected position's residual support is non-empty,
  // else (bonus position, or empty support) the target-law draw
  const unsigned long long key = (a < B - 1 && kr != 0ull) ? kr : kf;
  const int32_t tok = (int32_t)argmax_index(key);
  accept_len[s] = a;
  out_token[s] = tok;
  if (anchor_out) anchor_out[s] = tok;
}

}  // namespace

int sampling_splits(int vocab) { return (vocab + kSplit - 1) / kSplit; }

namespace {
// Splits of the emitted row in the residual pass at IT*4*kThreads logits each.
int residual_splits(int vocab, int it) {
  const int n = it * 4 * kThreads;
  return (vocab + n - 1) / n;
}
}  // namespace

int64_t sample_ws_bytes(int rows, int vocab) {
  return (int64_t)rows * sampling_splits(vocab) * (int64_t)sizeof(SplitStat);
}

namespace {
struct VerifyWs {
  int64_t stats, keys, acc, total;
};
VerifyWs verify_ws(int batch, int block, int vocab) {
  const int64_t ns = sampling_splits(vocab);
  const int64_t rows = (int64_t)batch * block + (int64_t)batch * (block - 1);
  auto al = [](int64_t x) { return ((x + 255) / 256) * 256; };
  VerifyWs w{};
  w.stats = 0;
  w.keys = al(rows * ns * (int64_t)sizeof(SplitStat));
  w.acc = w.keys + al((int64_t)batch * residual_splits(vocab, 1) * 16);
  w.total = w.acc + al((int64_t)batch * 4);
  return w;
}
}  // namespace

int64_t verify_ws_bytes(int batch, int block, int vocab) { return verify_ws(batch, block, vocab).total; }

hipError_t launch_sample_drafts(const float* logits, int64_t ld, int rows, int vocab, float temp,
                                uint64_t seed, int rnd, int32_t* tokens, float* logq, void* ws,
                                hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  const int ns = sampling_splits(vocab);
  SplitStat* part = reinterpret_cast<SplitStat*>(ws);
  const float inv_t = 1.0f / temp;
  hipLaunchKernelGGL(sample_split_kernel, dim3(ns, rows), dim3(kThreads), 0, st, logits, ld, vocab,
                     inv_t, seed, rnd, part, ns);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sample_finish_kernel, dim3((rows + 63) / 64), dim3(64), 0, st, logits, ld,
                     inv_t, part, ns, rows, tokens, logq);
  return hipGetLastError();
}

hipError_t launch_verify_sampled(const int32_t* drafts, const float* draft_logits,
                                 const float* draft_logq, const float* target_logits, int batch,
                                 int block, int vocab, float temp, uint64_t seed, int rnd,
                                 int32_t* accept_len, int32_t* out_token, int32_t* anchor_out,
                                 void* ws, hipStream_t st) {
  if (batch <= 0) return hipSuccess;
  const int ns = sampling_splits(vocab);
  const float inv_t = 1.0f / temp;
  char* w = reinterpret_cast<char*>(ws);
  const VerifyWs L = verify_ws(batch, block, vocab);
  // target rows, then (without log q) the draft rows
  const int64_t stats_rows = (int64_t)batch * block + (draft_logq ? 0 : (int64_t)batch * (block - 1));
  SplitStat* stats = reinterpret_cast<SplitStat*>(w + L.stats);
  unsigned long long* keys = reinterpret_cast<unsigned long long*>(w + L.keys);
  int32_t* acc = reinterpret_cast<int32_t*>(w + L.acc);
  hipLaunchKernelGGL(verify_stats_kernel, dim3(ns, (unsigned)stats_rows), dim3(kThreads), 0, st,
                     draft_logits, target_logits, batch, block, vocab, inv_t, stats, ns);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // The residual pass covers one row per sequence: few sequences take finer
  // splits (2048 or 1024 logits) so that the pass still spreads over the CUs.
  const int it = (int64_t)batch * residual_splits(vocab, 8) >= 256 ? 8
                 : (int64_t)batch * residual_splits(vocab, 2) >= 256 ? 2 : 1;
  const int nres = residual_splits(vocab, it);
#define DF_RES(I)                                                                                \
  hipLaunchKernelGGL(verify_residual_kernel<I>, dim3(nres, batch), dim3(kThreads), 0, st, drafts, \
                     draft_logits, draft_logq, target_logits, batch, block, vocab, inv_t, seed,   \
                     rnd, stats, ns, keys, acc)
  if (it == 8) DF_RES(8);
  else if (it == 2) DF_RES(2);
  else DF_RES(1);
#undef DF_RES
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(verify_finish_kernel, dim3((batch + 63) / 64), dim3(64), 0, st, keys, nres,
                     batch, block, acc, accept_len, out_token, anchor_out);
  return hipGetLastError();
}

// ---- allocation-free drafting ------------------------------------------------
// The split statistics of dflash_sample_drafts_static live in this file-scope
// device array instead of a caller workspace. Each GPU the library runs on
// holds its own copy (at its own address) until the process ends. In host
// code `sample_scratch` names a host-side stand-in, never the device memory:
// the device address is taken once per device with hipGetSymbolAddress and
// only that address is handed to kernels.
constexpr int64_t kSampleScratchBytes = 256 * 1024;
static __device__ __align__(256) unsigned char sample_scratch[kSampleScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

int64_t sample_static_scratch_bytes() { return kSampleScratchBytes; }

hipError_t sample_static_scratch(void** out) {
  *out = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(sample_scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace dflash
