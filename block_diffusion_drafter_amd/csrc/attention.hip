// KV-injected attention of the draft block over [cached context ; block] keys.
//
// The block's queries (B <= 16 rows per head) attend non-causally to every
// cached context position of their sequence plus the block's own keys, which
// the QKV step has already staged in the cache's scratch positions
// [ctx_len, ctx_len + B). With 16 queries per head over thousands of keys the
// work is a stream of the K/V cache, split over key chunks:
//
//   attn_partial: per KV head, the keys of all sequences are laid end to end
//     in 32-key blocks (sequence order) and split into equal ranges, one per
//     workgroup, so ragged batches keep every workgroup equally busy; a
//     workgroup runs each sequence segment of its range in turn, one wave per
//     query head of the GQA group. In bf16 the group's waves share each
//     32-key K/V block through an LDS ring filled by direct global->LDS loads
//     (every position crosses the memory system once, several blocks in
//     flight); the fp32 path loads per wave into registers. Scores are computed transposed, S^T = K Q^T (keys as
//     MFMA rows, queries as columns), and the output likewise, O^T = V^T P^T,
//     so each lane owns one query column: the online-softmax running max/sum
//     are per-lane values plus a two-step shuffle across the four lane groups.
//     P leaves the S^T accumulator already in the layout the next MFMA's B
//     operand needs (the key order inside a 32-key block is permuted to make
//     that so). V is stored channel-major inside 32-position blocks, so each
//     lane's V fragment is one 16-byte load. The next block's K/V is loaded
//     while the current one is multiplied. A sequence that lies within one
//     workgroup's range is normalised and written directly; otherwise each
//     segment's (max, sum, unnormalised O) goes to a partial buffer.
//   attn_combine: merges the segments of the sequences that span several
//     workgroups.
#include <climits>
#include <type_traits>

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

__device__ __forceinline__ int seq_ctx(const AttnArgs& p, int s) {
  const int cl = p.ctx_len[s];
  return cl < 0 ? 0 : cl;
}

__device__ __forceinline__ int seq_keys(const AttnArgs& p, int s) {
  return min(seq_ctx(p, s) + p.block, p.cap);
}

// First key position a layer reads for sequence s: 0, or in a sliding-window
// layer the 32-key block holding the oldest position query 0 sees
// (ctx_len - window + 1); positions below a query's own window edge inside
// that block are masked per query.
__device__ __forceinline__ int seq_first(const AttnArgs& p, int s) {
  if (p.window <= 0) return 0;
  const int lo = seq_ctx(p, s) - p.window + 1;
  return lo <= 0 ? 0 : (lo & ~31);
}

// Lowest key position query row r of sequence s may see (none below it).
__device__ __forceinline__ int query_first(const AttnArgs& p, int s, int r) {
  return p.window > 0 ? seq_ctx(p, s) + r - p.window + 1 : INT_MIN;
}

// First 32-key block of every sequence when one KV head's keys are laid end
// to end: pre[s] = sum over t < s of the blocks sequence t reads (from
// seq_first to its last key), pre[batch] = the total. Built in LDS by wave 0 (one load per lane and sequence, a wave scan
// per 64 sequences); every thread returns after the barrier that publishes it.
__device__ __forceinline__ void seq_block_prefix(const AttnArgs& p, int* pre) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int carry = 0;
    for (int base = 0; base < p.batch; base += 64) {
      const int s = base + lane;
      int v = s < p.batch ? (seq_keys(p, s) - seq_first(p, s) + 31) >> 5 : 0;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(v, o);
        if (lane >= o) v += u;
      }
      if (lane == 0) pre[base] = carry;
      if (s < p.batch) pre[s + 1] = carry + v;
      carry += __shfl(v, 63);
    }
    if (p.batch == 0 && lane == 0) pre[0] = 0;
  }
  __syncthreads();
}

// The equal split of one KV head's keys: tb 32-key blocks in total, of which
// workgroup w < nw takes [begin(w), begin(w + 1)). nw is the number of
// workgroups per head, capped so that each gets >= min_blocks blocks; both
// attention kernels derive the same split from ctx_len.
struct KeySplit {
  int tb, nw;
  __device__ int begin(int w) const { return (int)(((long long)w * tb) / nw); }
  // The workgroup whose range holds block b.
  __device__ int owner(int b) const { return (int)(((long long)(b + 1) * nw - 1) / tb); }
};

__device__ __forceinline__ KeySplit key_split(const AttnArgs& p, const int* pre) {
  const int tb = pre[p.batch];
  const int want = (tb + p.min_blocks - 1) / p.min_blocks;
  return KeySplit{tb, max(1, min(p.wg_per_head, want))};
}

// Partial entry of sequence s's segment in workgroup w (KV head g): w + s is
// unique over the (s, w) pairs that overlap, and below wg_per_head + batch.
__device__ __forceinline__ size_t part_entry(const AttnArgs& p, int g, int w, int s) {
  return (size_t)g * (p.wg_per_head + p.batch) + w + s;
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

// Online-softmax update of one wave's state with one 32-key block whose
// K/V fragments are in registers: S^T = K Q^T, running max / sum per query
// column (lane), O^T = alpha O^T + V^T P^T.
template <typename T, int HD>
struct AttnState {
  static constexpr int NDT = HD / 16;
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[NDT];
};

template <typename T, int HD>
__device__ __forceinline__ void attn_update(AttnState<T, HD>& S, const KVBlock<T, HD>& b,
                                            const u32x4* qf, int kb, int k_hi, int k_min,
                                            float scale_log2, int grp) {
  using KB = KVBlock<T, HD>;
  constexpr int FR = KB::FR, NDT = KB::NDT;
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
      const float v = (key < k_hi && key >= k_min) ? st[t][i] * scale_log2 : -INFINITY;
      st[t][i] = v;
      mx = fmaxf(mx, v);
    }
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  // A block may hold no key this query sees yet (sliding window): m_new stays
  // -inf, and a finite reference keeps alpha at 1 and every p at 0.
  const float m_new = fmaxf(S.m_run, mx);
  const float m_ref = m_new == -INFINITY ? 0.f : m_new;
  const float alpha = exp2f(S.m_run - m_ref);
  S.m_run = m_new;
  float psum = 0.f;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pv = exp2f(st[t][i] - m_ref);
      st[t][i] = pv;
      psum += pv;
    }
  S.l_run = S.l_run * alpha + psum;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) S.o[dt] *= alpha;
  if constexpr (sizeof(T) == 2) {
    bf16x8 pb;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) pb[4 * t + i] = (bf16)st[t][i];
    const u32x4 pf = __builtin_bit_cast(u32x4, pb);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) S.o[dt] = mfma_frag<T>(b.v[dt][0], pf, S.o[dt]);
  } else {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const u32x4 pf = __builtin_bit_cast(u32x4, st[t]);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) S.o[dt] = mfma_frag<T>(b.v[dt][t], pf, S.o[dt]);
    }
  }
}

// One 32-key block's online-softmax update of a wave's state, bf16 (the
// decoding kernel's and the packed-block kernel's). Scores outside
// [k_min, k_hi) are masked (a handful of compares). The softmax reference max
// moves only when a block exceeds it by more than 2^8 (lazy rescale: the
// probabilities stay <= 256, exact for the final normalisation, and the output
// accumulators are rarely touched outside the MFMAs). P enters the PV product
// as the sum of two bf16 parts (16 significant bits), so the products are as
// exact as the fp32 sum of probabilities they are normalised by; the second
// MFMA per tile is free where the kernel waits on memory. SPLIT = false keeps
// P's high part only (8 significant bits, as training attention kernels do),
// a third fewer MFMAs where the kernel waits on them instead.
template <int HD, bool SPLIT = true>
__device__ __forceinline__ void attn_update_lazy(AttnState<bf16, HD>& S,
                                                 const KVBlock<bf16, HD>& b, const u32x4* qf,
                                                 int kb, int k_hi, int k_min, float scale_log2,
                                                 int grp) {
  using T = bf16;
  constexpr int FR = KVBlock<T, HD>::FR, NDT = KVBlock<T, HD>::NDT;
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
      const float v = (key < k_hi && key >= k_min) ? st[t][i] * scale_log2 : -INFINITY;
      st[t][i] = v;
      mx = fmaxf(mx, v);
    }
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  if (__any(mx > S.m_run + 8.0f)) {
    const float m_new = fmaxf(S.m_run, mx);
    // m_new stays -inf while a query has seen no key (sliding window)
    const float alpha = m_new == -INFINITY ? 1.0f : exp2f(S.m_run - m_new);
    S.m_run = m_new;
    S.l_run *= alpha;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) S.o[dt] *= alpha;
  }
  const float m_ref = S.m_run == -INFINITY ? 0.f : S.m_run;
  float psum = 0.f;
  bf16x8 phi, plo;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // v_exp_f32: the argument is <= 8; tiny results may flush to 0
      const float pv = __builtin_amdgcn_exp2f(st[t][i] - m_ref);
      psum += pv;
      const bf16 hi = (bf16)pv;
      phi[4 * t + i] = hi;
      if constexpr (SPLIT) plo[4 * t + i] = (bf16)(pv - (float)hi);
    }
  S.l_run += psum;
  const u32x4 pf = __builtin_bit_cast(u32x4, phi);
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) S.o[dt] = mfma_frag<T>(b.v[dt][0], pf, S.o[dt]);
  if constexpr (SPLIT) {
    const u32x4 pl = __builtin_bit_cast(u32x4, plo);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) S.o[dt] = mfma_frag<T>(b.v[dt][0], pl, S.o[dt]);
  }
}

// The wave's Q fragments (same channel order as the K fragments).
template <typename T, int HD>
__device__ __forceinline__ void load_q(u32x4* qf, const AttnArgs& p, int s, int h, int r, int grp) {
  using KB = KVBlock<T, HD>;
  const T* qp = reinterpret_cast<const T*>(p.q) + (((size_t)s * p.n_heads + h) * 16 + r) * HD +
                grp * KB::EPF;
#pragma unroll
  for (int f = 0; f < KB::FR; ++f) qf[f] = ld16(qp + f * 4 * KB::EPF);
}

// End of a segment: a sequence that lies in one workgroup's range is
// normalised and written to the tiled output; otherwise (max, sum,
// unnormalised O) go to the segment's partial entry.
template <typename T, int HD>
__device__ __forceinline__ void attn_finish(AttnState<T, HD>& S, const AttnArgs& p, int s, int g,
                                            size_t entry, int j, int G, bool single, int r,
                                            int grp) {
  constexpr int NDT = HD / 16;
  const int h = g * G + j;
  S.l_run += __shfl_xor(S.l_run, 16);
  S.l_run += __shfl_xor(S.l_run, 32);
  if (single) {
    if (r < p.block) {
      // Four consecutive channels per lane and tile: contiguous in the tiled output.
      const float inv = 1.0f / S.l_run;
      T* out = reinterpret_cast<T*>(p.out);
      const int row = s * p.block + r;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        T* dst = out + tiled_index<T>(row, h * HD + 16 * dt + 4 * grp, p.out_nck);
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[i] = from_f32<T>(S.o[dt][i] * inv);
      }
    }
    return;
  }
  const size_t item = entry * G + j;
  if (grp == 0) {
    p.part_ml[(item * 16 + r) * 2 + 0] = S.m_run;
    p.part_ml[(item * 16 + r) * 2 + 1] = S.l_run;
  }
  float* po = p.part_o + item * HD * 16;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) po[(16 * dt + 4 * grp + i) * 16 + r] = S.o[dt][i];
}

// seg(s, k_lo, k_hi, single) for every sequence segment of workgroup w's
// range, in sequence order: keys [k_lo, k_hi) of sequence s; single when the
// segment is the whole sequence. The first sequence is found by binary search
// in the block prefix.
template <typename F>
__device__ __forceinline__ void for_each_segment(const AttnArgs& p, const int* pre,
                                                 const KeySplit& ks, int w, F&& seg) {
  const int b0 = ks.begin(w), b1 = ks.begin(w + 1);
  int lo = 0, hi = p.batch - 1;  // last s with pre[s] <= b0
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pre[mid] <= b0) lo = mid;
    else hi = mid - 1;
  }
  for (int s = lo; s < p.batch && pre[s] < b1; ++s) {
    const int bs = pre[s], be = pre[s + 1];
    const int n_keys = seq_keys(p, s), k0 = seq_first(p, s);
    const int a = max(b0, bs), b = min(b1, be);
    if (a < b) seg(s, k0 + 32 * (a - bs), min(n_keys, k0 + 32 * (b - bs)), a == bs && b == be);
  }
}

// fp32 path: each wave loads its K/V fragments straight into registers.
template <typename T, int HD>
__global__ __launch_bounds__(512) void attn_partial_kernel(AttnArgs p) {
  using KB = KVBlock<T, HD>;
  constexpr int FR = KB::FR, NDT = KB::NDT;
  const int lane = threadIdx.x & 63, j = threadIdx.x >> 6;
  const int r = lane & 15, grp = lane >> 4;
  const int w = blockIdx.x, g = blockIdx.y;
  const int G = p.n_heads / p.n_kv_heads;
  const int h = g * G + j;
  extern __shared__ int pre[];
  seq_block_prefix(p, pre);
  const KeySplit ks = key_split(p, pre);
  if (w >= ks.nw) return;
  for_each_segment(p, pre, ks, w, [&](int s, int k_lo, int k_hi, bool single) {
  const size_t kvoff = (size_t)(s * p.n_kv_heads + g) * p.cap * HD;
  const T* K = reinterpret_cast<const T*>(p.k) + kvoff;
  const T* V = reinterpret_cast<const T*>(p.v) + kvoff;

  const int k_min = query_first(p, s, r);
  u32x4 qf[FR];
  load_q<T, HD>(qf, p, s, h, r, grp);
  AttnState<T, HD> S;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) S.o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  if constexpr (HD == 64) {
    // Two blocks in flight: the next block's K/V loads while this one is used.
    KB b0, b1;
    load_block<T, HD>(b0, K, V, k_lo, k_hi, r, grp);
    for (int kb = k_lo; kb < k_hi; kb += 64) {
      const bool has1 = kb + 32 < k_hi;
      if (has1) load_block<T, HD>(b1, K, V, kb + 32, k_hi, r, grp);
      attn_update<T, HD>(S, b0, qf, kb, k_hi, k_min, p.scale_log2, grp);
      if (has1) {
        if (kb + 64 < k_hi) load_block<T, HD>(b0, K, V, kb + 64, k_hi, r, grp);
        attn_update<T, HD>(S, b1, qf, kb + 32, k_hi, k_min, p.scale_log2, grp);
      }
    }
  } else {
    // head_dim 128: one block of fragments already fills the registers.
    for (int kb = k_lo; kb < k_hi; kb += 32) {
      KB b0;
      load_block<T, HD>(b0, K, V, kb, k_hi, r, grp);
      attn_update<T, HD>(S, b0, qf, kb, k_hi, k_min, p.scale_log2, grp);
    }
  }
  attn_finish<T, HD>(S, p, s, g, part_entry(p, g, w, s), j, G, single, r, grp);
  });
}

typedef __attribute__((address_space(3))) void* attn_lds_ptr;
typedef const __attribute__((address_space(1))) void* attn_gbl_ptr;

// Wait until at most N of this wave's global->LDS loads are outstanding and
// its LDS reads have returned, then meet the other waves of the group.
template <int N>
__device__ __forceinline__ void attn_wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// bf16 path: the G waves of a KV group share each 32-key K/V block through an
// LDS ring. A block is NI = HD/8 wave-wide 1 KB fragments (2*FR of K, NDT of
// V), copied by direct global->LDS loads split over the waves; each load's
// lanes gather exactly the 16-byte pieces the MFMA operand layout wants, so a
// wave reads every fragment back as 64 lanes x 16 contiguous bytes. NSB ring
// slots keep NSB-1 blocks in flight per group with no staging registers.
// Every step issues a block (past the end: the last one again, into a slot
// nobody reads any more), so the wait counts are constants and the loop has
// no branches; only the sequence's final block (a partial one) and
// sliding-window layers apply the key masks. The softmax rescale is lazy: the running reference max moves
// only when a block's max exceeds it by more than 2^8 (probabilities stay
// <= 256, exact for the final normalisation), so the output accumulators are
// rarely touched outside the MFMAs.
template <int HD, int G, int NSB = 4, int HPG = 1>
__global__ __launch_bounds__(64 * G * HPG) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_partial_lds_kernel(AttnArgs p) {
  using T = bf16;
  using KB = KVBlock<T, HD>;
  constexpr int EPF = KB::EPF, FR = KB::FR, NDT = KB::NDT;
  constexpr int NI = 2 * FR + NDT;  // fragments per block
  constexpr int IPW = NI / G;       // fragments each wave copies per block
  static_assert(NI % G == 0, "block fragments must split evenly over the group");
  static_assert(NSB >= 3, "a slot being read, one arriving, one being filled");
  __shared__ u32x4 ring_all[HPG][NSB][NI][64];

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = wv % G, hg = wv / G;  // wave j of the workgroup's head group hg
  const int r = lane & 15, grp = lane >> 4;
  const int w = blockIdx.x, g = blockIdx.y * HPG + hg;
  const int h = g * G + j;
  auto& ring = ring_all[hg];
  extern __shared__ int pre[];
  seq_block_prefix(p, pre);
  const KeySplit ks = key_split(p, pre);
  if (w >= ks.nw) return;
  bool first = true;
  for_each_segment(p, pre, ks, w, [&](int s, int k_lo, int k_hi, bool single) {
  // The previous segment's last ring reads are done in every wave before its
  // slots are refilled.
  if (!first) __syncthreads();
  first = false;
  const int nblk = (k_hi - k_lo + 31) / 32;

  const size_t kvoff = (size_t)(s * p.n_kv_heads + g) * p.cap * HD;
  const T* K = reinterpret_cast<const T*>(p.k) + kvoff;
  const T* V = reinterpret_cast<const T*>(p.v) + kvoff;

  // Fragment i of block n (key base kb = k_lo + 32 n, a multiple of 32 below
  // cap, so every address stays inside the sequence's cache rows): i < 2*FR
  // is K tile i/FR, fragment i%FR: lane (r, grp) takes key kb + key_of(t, r),
  // channels [4*EPF*f + EPF*grp, +EPF). Else V channel tile dt = i - 2*FR:
  // lane (r, grp) takes channel 16 dt + r, keys 8 grp .. 8 grp + 7 of the
  // block. Either way block n's fragment is block 0's plus n * 32 * HD
  // elements, so each wave's sources are set up once per segment.
  const T* src[IPW];
#pragma unroll
  for (int u = 0; u < IPW; ++u) {
    const int i = j + G * u;
    if (i < 2 * FR) {
      const int t = i / FR, f = i % FR;
      src[u] = K + (size_t)(k_lo + key_of<T>(t, r)) * HD + f * 4 * EPF + grp * EPF;
    } else {
      const int dt = i - 2 * FR;
      src[u] = V + (size_t)(k_lo / kKeyBlock) * HD * kKeyBlock + (16 * dt + r) * kKeyBlock + 8 * grp;
    }
  }
  auto issue = [&](int n, int slot) {
#pragma unroll
    for (int u = 0; u < IPW; ++u)
      __builtin_amdgcn_global_load_lds((attn_gbl_ptr)(src[u] + (size_t)n * 32 * HD),
                                       (attn_lds_ptr)&ring[slot][j + G * u][0], 16, 0, 0);
  };
  auto read_block = [&](KB& b, int slot) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int f = 0; f < FR; ++f) b.k[t][f] = ring[slot][t * FR + f][lane];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) b.v[dt][0] = ring[slot][2 * FR + dt][lane];
  };

  const int k_min = query_first(p, s, r);
  u32x4 qf[FR];
  load_q<T, HD>(qf, p, s, h, r, grp);
  // Consume Q here, so the compiler's wait for it happens before the ring's
  // loads are issued (later, it would have to drain the whole ring).
#pragma unroll
  for (int f = 0; f < FR; ++f) asm volatile("" ::"v"(qf[f]));
  AttnState<T, HD> S;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) S.o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto update = [&](const KB& b, int n) {
    attn_update_lazy<HD>(S, b, qf, k_lo + 32 * n, k_hi, k_min, p.scale_log2, grp);
  };

  // Block n: wait until it has landed and every wave is done with block n-1,
  // refill block n-1's slot with block n-1+NSB, read block n from LDS and
  // multiply it (the other waves on the SIMD cover the LDS latency).
  // A segment of at most NSB blocks is loaded whole and waited for once;
  // longer ones run the ring.
  const bool whole = nblk <= NSB;
#pragma unroll
  for (int n = 0; n < NSB; ++n)
    if (!whole || n < nblk) issue(min(n, nblk - 1), n);
  if (whole) attn_wait_barrier<0>();
  else attn_wait_barrier<IPW * (NSB - 1)>();
  KB b;
  for (int n = 0; n < nblk; ++n) {
    if (n > 0 && !whole) {
      attn_wait_barrier<IPW * (NSB - 2)>();
      issue(min(n - 1 + NSB, nblk - 1), (n - 1) % NSB);
    }
    read_block(b, n % NSB);
    if (n == nblk - 1 && k_lo + 32 * n + 32 > k_hi) {
      // Positions past the last key may hold anything (even NaN bit
      // patterns); their probabilities are 0, so their values must be 0 too.
      const int kb = k_lo + 32 * n;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) b.v[dt][0] = keep_first<T>(b.v[dt][0], k_hi - (kb + 8 * grp));
    }
    update(b, n);
  }
  // The ring's trailing loads land before its slots are reused (or the
  // workgroup's LDS is released).
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  attn_finish<T, HD>(S, p, s, g, part_entry(p, g, w, s), j, G, single, r, grp);
  });
}

// Merge of the segment partials of the sequences that span several
// workgroups: one workgroup per (KV head, sequence, channel slice), one wave
// per query head of the group; lane (q, c) owns query q and CPL consecutive
// channels of the slice (4 * CPL channels). The block prefix is built once
// per workgroup and a sequence in one piece returns at once. Every lane reads
// the segments' (max, sum) of its query, then their partial outputs, in
// segment order (loads independent of each other), and writes its normalised
// channels. Few (KV head, sequence) pairs with many segments each (batch 1)
// take narrow slices, so more workgroups share the reads.
template <typename T, int HD, int CPL>
__global__ __launch_bounds__(512) void attn_combine_kernel(AttnArgs p) {
  const int g = blockIdx.x, s = blockIdx.y, slice = blockIdx.z;
  const int G = p.n_heads / p.n_kv_heads;
  extern __shared__ int pre[];
  seq_block_prefix(p, pre);
  const KeySplit ks = key_split(p, pre);
  const int w0 = ks.owner(pre[s]), w1 = ks.owner(pre[s + 1] - 1);
  if (w0 == w1) return;  // one segment: written by the partial kernel
  const int nch = w1 - w0 + 1;
  const int t = threadIdx.x, j = t >> 6, q = t & 15, c = (t >> 4) & 3;
  if (q >= p.block) return;
  const size_t e0 = part_entry(p, g, w0, s);  // segment k is entry e0 + k
  const int ch0 = 4 * CPL * slice + CPL * c;
  // Segments in groups of four: every load of a group (each segment's max,
  // sum and partial channels) goes out at once, then the group is merged
  // into the running (max, sum, output), rescaled to the new max.
  constexpr int KG = 4;
  float M = -INFINITY, L = 0.f, o[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) o[i] = 0.f;
  for (int k0 = 0; k0 < nch; k0 += KG) {
    float mk[KG], lk[KG], ok[KG][CPL];
#pragma unroll
    for (int u = 0; u < KG; ++u) {
      const bool ok_k = k0 + u < nch;
      const size_t item = (e0 + min(k0 + u, nch - 1)) * G + j;
      const float* po = p.part_o + (item * HD + ch0) * 16 + q;
      mk[u] = ok_k ? p.part_ml[(item * 16 + q) * 2] : -INFINITY;
      lk[u] = ok_k ? p.part_ml[(item * 16 + q) * 2 + 1] : 0.f;
#pragma unroll
      for (int i = 0; i < CPL; ++i) ok[u][i] = ok_k ? po[i * 16] : 0.f;
    }
    float Mn = M;
#pragma unroll
    for (int u = 0; u < KG; ++u) Mn = fmaxf(Mn, mk[u]);
    // A sequence whose queries saw no key yet (sliding window) keeps -inf.
    const float ref = Mn == -INFINITY ? 0.f : Mn;
    const float a = exp2f(M - ref);
    L *= a;
#pragma unroll
    for (int i = 0; i < CPL; ++i) o[i] *= a;
#pragma unroll
    for (int u = 0; u < KG; ++u) {
      const float wk = exp2f(mk[u] - ref);
      L += lk[u] * wk;
#pragma unroll
      for (int i = 0; i < CPL; ++i) o[i] += ok[u][i] * wk;
    }
    M = Mn;
  }
  const float inv = 1.0f / L;
  T* out = reinterpret_cast<T*>(p.out);
  const int row = s * p.block + q, h = g * G + j;
#pragma unroll
  for (int i = 0; i < CPL; ++i)
    out[tiled_index<T>(row, h * HD + ch0 + i, p.out_nck)] = from_f32<T>(o[i] * inv);
}

// Many segments per sequence (batch 1-4): merge of the segment partials of
// one (query head, sequence, 16-channel
// slice). Thread (q, cg) owns query row q and the segments c = cg, cg + 16,
// ...: it reduces the row's running max and sum over its segments, the 16
// threads of a row combine them through LDS, then each thread accumulates its
// segments' weighted partial outputs for the slice's 16 channels and LDS sums
// the 16 segment groups. Every thread's loads are independent of each other.
template <typename T, int HD>
__global__ __launch_bounds__(256) void attn_combine_chunks_kernel(AttnArgs p) {
  __shared__ float red_m[16][17], red_l[16][17];
  __shared__ float red_o[16][16][17];
  const int h = blockIdx.x, s = blockIdx.y, slice = blockIdx.z;
  const int G = p.n_heads / p.n_kv_heads;
  const int g = h / G, j = h % G;
  extern __shared__ int pre[];
  seq_block_prefix(p, pre);
  const KeySplit ks = key_split(p, pre);
  const int w0 = ks.owner(pre[s]), w1 = ks.owner(pre[s + 1] - 1);
  if (w0 == w1) return;  // one segment: written by the partial kernel
  // Segments c = 0 .. nch-1 come from workgroups w0 + c (every one in between
  // has a non-empty range since nw <= tb), at entries w0 + c + s.
  const int nch = w1 - w0 + 1;
  const int t = threadIdx.x, q = t & 15, cg = t >> 4;
  const size_t item0 = part_entry(p, g, w0, s) * G + j;
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
  dim3 grid(a.wg_per_head, a.n_kv_heads, 1);
  const size_t pre_bytes = (size_t)(a.batch + 1) * sizeof(int);  // block prefix in LDS
  if constexpr (sizeof(T) == 2) {
    switch (G) {
      case 1: hipLaunchKernelGGL((attn_partial_lds_kernel<HD, 1>), grid, dim3(64), pre_bytes, st, a); break;
      case 2: hipLaunchKernelGGL((attn_partial_lds_kernel<HD, 2>), grid, dim3(128), pre_bytes, st, a); break;
      case 4:
        // Two KV heads per workgroup (one per group of four waves): the
        // launch is one workgroup per CU, all dispatched at once, instead of
        // two per CU of which the later-dispatched one finishes last.
        if (a.n_kv_heads % 2 == 0)
          hipLaunchKernelGGL((attn_partial_lds_kernel<HD, 4, 4, 2>),
                             dim3(a.wg_per_head, a.n_kv_heads / 2, 1), dim3(512), pre_bytes, st, a);
        else
          hipLaunchKernelGGL((attn_partial_lds_kernel<HD, 4>), grid, dim3(256), pre_bytes, st, a);
        break;
      case 8: hipLaunchKernelGGL((attn_partial_lds_kernel<HD, 8>), grid, dim3(512), pre_bytes, st, a); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    hipLaunchKernelGGL((attn_partial_kernel<T, HD>), grid, dim3(64 * G), pre_bytes, st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.wg_per_head <= 1) return e;
  prof_end(st);
  prof_begin(DFLASH_K_ATTN_COMBINE, 0.0, 0.0, st);
  if (a.n_kv_heads * a.batch >= 64)
    hipLaunchKernelGGL((attn_combine_kernel<T, HD, 8>), dim3(a.n_kv_heads, a.batch, HD / 32),
                       dim3(64 * G), pre_bytes, st, a);
  else
    hipLaunchKernelGGL((attn_combine_chunks_kernel<T, HD>), dim3(a.n_heads, a.batch, HD / 16),
                       dim3(256), pre_bytes, st, a);
  return hipGetLastError();
}

// Training-pattern attention of packed blocks: one workgroup per (block,
// KV head), one wave per query head of the group. The block's context is the
// prefix 0 .. anchor-1 of its sequence's cache, streamed as in the decoding
// kernel's register path with two 32-key blocks in flight (many blocks of a
// sequence read the same prefix, which stays in L2); then the block's own B
// keys, gathered from the packed K/V into one masked 32-key block. Anchors
// outside [0, min(ctx_len, cap)] are clamped and flag DFLASH_DEV_CAPACITY.
template <typename T, int HD>
__global__ __launch_bounds__(512) void packed_attn_kernel(PackedAttnArgs p) {
  using KB = KVBlock<T, HD>;
  constexpr int EPF = KB::EPF, FR = KB::FR, NDT = KB::NDT;
  const int lane = threadIdx.x & 63, j = threadIdx.x >> 6;
  const int r = lane & 15, grp = lane >> 4;
  const int blk = blockIdx.x, g = blockIdx.y;
  const int G = p.n_heads / p.n_kv_heads, Hq = p.n_heads, Hkv = p.n_kv_heads;
  const int h = g * G + j, B = p.block;
  const int s = blk / p.blocks_per_seq;
  int a = p.anchors[blk];
  const int lim = min(max(p.ctx_len[s], 0), p.cap);
  if (a < 0 || a > lim) {
    if (threadIdx.x == 0 && g == 0 && p.dev_status) atomicOr(p.dev_status, DFLASH_DEV_CAPACITY);
    a = a < 0 ? 0 : lim;
  }

  // Q fragments of query row r (zero past the block), channel order as K.
  u32x4 qf[FR];
  {
    const T* qp = reinterpret_cast<const T*>(p.q) + (((size_t)blk * B + r) * Hq + h) * HD + grp * EPF;
#pragma unroll
    for (int f = 0; f < FR; ++f) qf[f] = r < B ? ld16(qp + f * 4 * EPF) : zero16();
  }
  AttnState<T, HD> S;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) S.o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const size_t kvoff = (size_t)(s * Hkv + g) * p.cap * HD;
  const T* K = reinterpret_cast<const T*>(p.k) + kvoff;
  const T* V = reinterpret_cast<const T*>(p.v) + kvoff;
  if (a > 0 && sizeof(T) == 4 && HD == 128) {
    // fp32 at head_dim 128: one block of fragments already fills the registers
    for (int kb = 0; kb < a; kb += 32) {
      KB b0;
      load_block<T, HD>(b0, K, V, kb, a, r, grp);
      attn_update<T, HD>(S, b0, qf, kb, a, INT_MIN, p.scale_log2, grp);
    }
  } else if (a > 0) {
    KB b0, b1;
    load_block<T, HD>(b0, K, V, 0, a, r, grp);
    for (int kb = 0; kb < a; kb += 64) {
      const bool has1 = kb + 32 < a;
      if (has1) load_block<T, HD>(b1, K, V, kb + 32, a, r, grp);
      attn_update<T, HD>(S, b0, qf, kb, a, INT_MIN, p.scale_log2, grp);
      if (has1) {
        if (kb + 64 < a) load_block<T, HD>(b0, K, V, kb + 64, a, r, grp);
        attn_update<T, HD>(S, b1, qf, kb + 32, a, INT_MIN, p.scale_log2, grp);
      }
    }
  }

  // The block's own keys as one 32-key block: key k < B of the block at the
  // fragment positions the decoding layout gives key k; the rest zero (their
  // scores are masked, their values must be 0).
  {
    KB b;
    const T* kp = reinterpret_cast<const T*>(p.k_blk);
    const T* vp = reinterpret_cast<const T*>(p.v_blk);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int key = key_of<T>(t, r);
      const T* src = kp + (((size_t)blk * B + key) * Hkv + g) * HD + grp * EPF;
#pragma unroll
      for (int f = 0; f < FR; ++f) b.k[t][f] = key < B ? ld16(src + f * 4 * EPF) : zero16();
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const int ch = 16 * dt + r;
#pragma unroll
      for (int u = 0; u < KB::VF; ++u) {
        // the decoding layout's V fragment: keys koff .. koff + EPF - 1 of channel ch
        const int koff = (sizeof(T) == 2) ? 8 * grp : 16 * u + 4 * grp;
        T vals[EPF];
#pragma unroll
        for (int e = 0; e < EPF; ++e) {
          const int key = koff + e;
          vals[e] = key < B ? vp[(((size_t)blk * B + key) * Hkv + g) * HD + ch] : from_f32<T>(0.f);
        }
        b.v[dt][u] = *reinterpret_cast<const u32x4*>(vals);
      }
    }
    attn_update<T, HD>(S, b, qf, 0, B, INT_MIN, p.scale_log2, grp);
  }

  // Normalise and write query rows r < B: lane (r, grp) holds channels
  // 16 dt + 4 grp + i.
  S.l_run += __shfl_xor(S.l_run, 16);
  S.l_run += __shfl_xor(S.l_run, 32);
  if (r < B) {
    const float inv = 1.0f / S.l_run;
    T* out = reinterpret_cast<T*>(p.out) + (((size_t)blk * B + r) * Hq + h) * HD;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) out[16 * dt + 4 * grp + i] = from_f32<T>(S.o[dt][i] * inv);
  }
}

// bf16 training-pattern attention, query tiles over several blocks: one
// workgroup per (TB consecutive blocks of a sequence, KV head), one wave per
// query head of the group holding the TB blocks' queries (TB states). The
// context prefix up to the tile's largest anchor streams once through an
// LDS ring (direct global->LDS loads, as in the decoding kernel) and every
// 32-key block updates each of the tile's blocks whose anchor lies past its
// start (keys at or after a block's anchor masked). Blocks drawn in anchor
// order share most of their prefix, so one stream serves TB blocks: TB times
// fewer K/V reads and TB times the matrix work per LDS read. Then each block
// attends to its own B keys, gathered from the packed K/V.
template <int HD, int G, int TB, int NSB = 4>
__global__ __launch_bounds__(64 * G) __attribute__((amdgpu_waves_per_eu(TB <= 2 ? 2 : 1, TB <= 2 ? 2 : 1)))
void packed_attn_tile_kernel(PackedAttnArgs p, int tiles_per_seq) {
  using T = bf16;
  using KB = KVBlock<T, HD>;
  constexpr int EPF = KB::EPF, FR = KB::FR, NDT = KB::NDT;
  constexpr int NI = 2 * FR + NDT;
  constexpr int IPW = NI / G;
  static_assert(NI % G == 0, "block fragments must split evenly over the group");
  __shared__ u32x4 ring[NSB][NI][64];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, grp = lane >> 4;
  const int Hq = p.n_heads, Hkv = p.n_kv_heads, B = p.block;
  // Workgroup -> (sequence, KV head) pair and tile. The dispatcher deals
  // workgroups round-robin to the 8 XCDs (each with its own L2); when the
  // pairs split evenly over them, XCD x takes pairs x*n/8 .. (x+1)*n/8 - 1,
  // their tiles in order, so the context prefix the tiles of one pair share is
  // fetched into one L2 instead of all eight.
  const int n_pairs = (p.n_blk / p.blocks_per_seq) * Hkv;
  int pair, tile;
  if (n_pairs % 8 == 0) {
    const int xcd = blockIdx.x & 7, q = blockIdx.x >> 3;
    pair = xcd * (n_pairs / 8) + q / tiles_per_seq;
    tile = q % tiles_per_seq;
  } else {
    pair = blockIdx.x / tiles_per_seq;
    tile = blockIdx.x % tiles_per_seq;
  }
  const int g = pair % Hkv;
  const int h = g * G + w;
  const int s = pair / Hkv, j0 = tile * TB;
  const int nt = min(TB, p.blocks_per_seq - j0);
  const int blk0 = s * p.blocks_per_seq + j0;
  const int lim = min(max(p.ctx_len[s], 0), p.cap);
  int a[TB];
  int kmax = 0;
#pragma unroll
  for (int t = 0; t < TB; ++t) {
    a[t] = 0;
    if (t < nt) {
      int v = p.anchors[blk0 + t];
      if (v < 0 || v > lim) {
        if (threadIdx.x == 0 && g == 0 && p.dev_status) atomicOr(p.dev_status, DFLASH_DEV_CAPACITY);
        v = v < 0 ? 0 : lim;
      }
      a[t] = v;
      kmax = max(kmax, v);
    }
  }

  u32x4 qf[TB][FR];
  AttnState<T, HD> S[TB];
#pragma unroll
  for (int t = 0; t < TB; ++t) {
    const T* qp = reinterpret_cast<const T*>(p.q) + (((size_t)(blk0 + t) * B + r) * Hq + h) * HD + grp * EPF;
#pragma unroll
    for (int f = 0; f < FR; ++f) qf[t][f] = (t < nt && r < B) ? ld16(qp + f * 4 * EPF) : zero16();
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) S[t].o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int t = 0; t < TB; ++t)
#pragma unroll
    for (int f = 0; f < FR; ++f) asm volatile("" ::"v"(qf[t][f]));

  // Context blocks 0 .. nblk-1 through the ring; fragment sources as in the
  // decoding kernel (block n = block 0 + n * 32 * HD elements).
  const int nblk = (kmax + 31) / 32;
  const size_t kvoff = (size_t)(s * Hkv + g) * p.cap * HD;
  const T* K = reinterpret_cast<const T*>(p.k) + kvoff;
  const T* V = reinterpret_cast<const T*>(p.v) + kvoff;
  if (nblk > 0) {
    const T* src[IPW];
#pragma unroll
    for (int u = 0; u < IPW; ++u) {
      const int i = w + G * u;
      if (i < 2 * FR) {
        const int t = i / FR, f = i % FR;
        src[u] = K + (size_t)key_of<T>(t, r) * HD + f * 4 * EPF + grp * EPF;
      } else {
        const int dt = i - 2 * FR;
        src[u] = V + (size_t)(16 * dt + r) * kKeyBlock + 8 * grp;
      }
    }
    auto issue = [&](int n, int slot) {
#pragma unroll
      for (int u = 0; u < IPW; ++u)
        __builtin_amdgcn_global_load_lds((attn_gbl_ptr)(src[u] + (size_t)n * 32 * HD),
                                         (attn_lds_ptr)&ring[slot][w + G * u][0], 16, 0, 0);
    };
    const bool whole = nblk <= NSB;
#pragma unroll
    for (int n = 0; n < NSB; ++n)
      if (!whole || n < nblk) issue(min(n, nblk - 1), n);
    if (whole) attn_wait_barrier<0>();
    else attn_wait_barrier<IPW * (NSB - 1)>();
    KB b;
    for (int n = 0; n < nblk; ++n) {
      if (n > 0 && !whole) {
        attn_wait_barrier<IPW * (NSB - 2)>();
        issue(min(n - 1 + NSB, nblk - 1), (n - 1) % NSB);
      }
      const int slot = n % NSB;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int f = 0; f < FR; ++f) b.k[t][f] = ring[slot][t * FR + f][lane];
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) b.v[dt][0] = ring[slot][2 * FR + dt][lane];
      const int kb = 32 * n;
      if (kb + 32 > kmax) {
        // positions past the largest anchor may lie past the context (cache
        // slack: anything, even NaN bit patterns); every block masks them
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) b.v[dt][0] = keep_first<T>(b.v[dt][0], kmax - (kb + 8 * grp));
      }
#pragma unroll
      for (int t = 0; t < TB; ++t)
        if (kb < a[t]) attn_update_lazy<HD, false>(S[t], b, qf[t], kb, a[t], INT_MIN, p.scale_log2, grp);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }

  // Each block's own keys as one masked 32-key block.
  const T* kp = reinterpret_cast<const T*>(p.k_blk);
  const T* vp = reinterpret_cast<const T*>(p.v_blk);
#pragma unroll
  for (int t = 0; t < TB; ++t) {
    if (t >= nt) break;
    const size_t bb = (size_t)(blk0 + t) * B;
    KB b;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int key = key_of<T>(u, r);
      const T* src = kp + ((bb + key) * Hkv + g) * HD + grp * EPF;
#pragma unroll
      for (int f = 0; f < FR; ++f) b.k[u][f] = key < B ? ld16(src + f * 4 * EPF) : zero16();
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      T vals[EPF];
#pragma unroll
      for (int e = 0; e < EPF; ++e) {
        const int key = 8 * grp + e;
        vals[e] = key < B ? vp[((bb + key) * Hkv + g) * HD + 16 * dt + r] : from_f32<T>(0.f);
      }
      b.v[dt][0] = *reinterpret_cast<const u32x4*>(vals);
    }
    attn_update_lazy<HD, false>(S[t], b, qf[t], 0, B, INT_MIN, p.scale_log2, grp);
  }

#pragma unroll
  for (int t = 0; t < TB; ++t) {
    if (t >= nt) break;
    float l = S[t].l_run;
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (r < B) {
      const float inv = 1.0f / l;
      T* out = reinterpret_cast<T*>(p.out) + (((size_t)(blk0 + t) * B + r) * Hq + h) * HD;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) out[16 * dt + 4 * grp + i] = from_f32<T>(S[t].o[dt][i] * inv);
    }
  }
}

template <int HD, int TB>
static hipError_t launch_packed_tile(const PackedAttnArgs& a, hipStream_t st) {
  const int G = a.n_heads / a.n_kv_heads;
  const int tiles = (a.blocks_per_seq + TB - 1) / TB;
  const dim3 grid((a.n_blk / a.blocks_per_seq) * tiles * a.n_kv_heads);
  switch (G) {
    case 1: hipLaunchKernelGGL((packed_attn_tile_kernel<HD, 1, TB>), grid, dim3(64), 0, st, a, tiles); break;
    case 2: hipLaunchKernelGGL((packed_attn_tile_kernel<HD, 2, TB>), grid, dim3(128), 0, st, a, tiles); break;
    case 4: hipLaunchKernelGGL((packed_attn_tile_kernel<HD, 4, TB>), grid, dim3(256), 0, st, a, tiles); break;
    case 8: hipLaunchKernelGGL((packed_attn_tile_kernel<HD, 8, TB>), grid, dim3(512), 0, st, a, tiles); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_packed_attention(int dtype, const PackedAttnArgs& a, hipStream_t st) {
  if (a.n_blk <= 0) return hipSuccess;
  const int G = a.n_heads / a.n_kv_heads;
  if (G > 8 || a.block < 1 || a.block > 16) return hipErrorInvalidValue;
  const dim3 grid(a.n_blk, a.n_kv_heads), block(64 * G);
  if (dtype == DFLASH_BF16) {
    // query tiles of 2 blocks: TB = 4 (one wave per SIMD) ran 1.8x slower, TB = 3 spills
    if (a.head_dim == 128) return launch_packed_tile<128, 2>(a, st);
    if (a.head_dim == 64) return launch_packed_tile<64, 2>(a, st);
    return hipErrorInvalidValue;
  } else {
    if (a.head_dim == 128) hipLaunchKernelGGL((packed_attn_kernel<float, 128>), grid, block, 0, st, a);
    else if (a.head_dim == 64) hipLaunchKernelGGL((packed_attn_kernel<float, 64>), grid, block, 0, st, a);
    else return hipErrorInvalidValue;
  }
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
