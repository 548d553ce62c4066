// MFMA-bound GEMM for batched drafting: Y = A · W^T with A [M, K] tiled
// activations (hundreds of rows) and W [N, K] tiled weights, bf16 in, fp32
// accumulation, the same fused epilogues as the weight-streaming kernel.
//
// At a few hundred rows every projection does ~400+ flops per weight byte,
// above the chip's ridge point, so the kernel is organised around the matrix
// cores:
//   * a workgroup owns a BM x BN output block (256x256 or 256x192 with 8
//     waves, 128x128 or 128x96 with 4, whichever fills the 256 CUs best for
//     the least work); each wave a (BM/WGM) x (BN/WGN) sub-block of 16x16
//     MFMA tiles held in registers;
//   * K advances in stages of 32 (8 waves) or 64 (4 waves). A stage of A
//     and W is copied from
//     the tiled layout into LDS unchanged by direct global->LDS loads
//     (global_load_lds_dwordx4: one 1 KB fragment per wave instruction, no
//     registers), and every LDS read of an MFMA operand is 64 lanes x 16
//     contiguous bytes (no bank conflicts, no shuffles);
//   * the stages form a ring of NS slots in LDS with NS-1 stages in flight;
//     one wait + barrier per stage (a register-staged double buffer left the
//     matrix cores idle on load latency at every stage); every wave reads
//     the next stage's operands into a second register set while it
//     multiplies the current ones;
//   * workgroups that share a column block but differ in row block are
//     numbered 8 apart, so they run on the same XCD at about the same time
//     and the second reads the weight block from that XCD's L2.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace dflash {

namespace {

constexpr int kEPF = 8;          // bf16 per 16-byte fragment
constexpr int kKC = 128;         // k per tiled chunk
constexpr int kFRAG = 64 * kEPF; // elements of one 1 KB wave-wide fragment

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef const __attribute__((address_space(1))) void* gbl_ptr_t;

// KF fragments per tile per stage (stage k = 32 KF), NS ring slots.
template <int BM, int BN, int WGM, int WGN, int KF, int NS>
struct MfmaGeom {
  static constexpr int NW = WGM * WGN;
  static constexpr int WM = BM / WGM, WN = BN / WGN;
  static constexpr int TM = WM / 16, TN = WN / 16;  // 16x16 tiles per wave
  static constexpr int AT = BM / 16, BT = BN / 16;  // row tiles of A / W in a block
  static constexpr int SF = (AT + BT) * KF;         // fragments per stage
  static constexpr int FPW = SF / NW;               // fragments each wave copies per stage
  static_assert(SF % NW == 0, "stage fragments must split evenly over the waves");
  static_assert(NS >= 2, "ring needs a slot being read and one arriving");
};

__device__ __forceinline__ int p_ksplit(const GemmArgs& p) { return p.ksplit > 1 ? p.ksplit : 1; }

// Wait until at most N of this wave's global->LDS loads are outstanding and
// all of its LDS reads have returned, then meet the other waves. The memory
// clobber keeps the compiler from moving LDS accesses across it.
template <int N>
__device__ __forceinline__ void wait_loads_and_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

}  // namespace

// resid[m, n] += acc over a wave's TM x TN tiles (lane (r, grp) holds rows
// 4*grp + e of column col0 + 16 j in tile (i, j)). All loads of a row of
// tiles go out before its stores: element by element, the compiler waited for
// every load, since a store might alias the next load.
template <int TM, int TN>
__device__ __forceinline__ void resid_add_tiles(const GemmArgs& p, const f32x4 (&acc)[TM][TN],
                                                int row0, int col0, int grp) {
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    float v[TN][4];
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = row0 + 16 * i + 4 * grp + e, n = col0 + 16 * j;
        v[j][e] = (m < p.M && n < p.N) ? p.resid[(int64_t)m * p.out_stride + n] : 0.f;
      }
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = row0 + 16 * i + 4 * grp + e, n = col0 + 16 * j;
        if (m < p.M && n < p.N) p.resid[(int64_t)m * p.out_stride + n] = v[j][e] + acc[i][j][e];
      }
  }
}

// Four waves, one per SIMD, for the narrow blocks (128 x 128 / 96): one
// workgroup per CU (the LDS ring takes most of it), each wave prefetching the
// next stage's operands into registers while it multiplies the current ones.
template <int BM, int BN, int WGM, int WGN, int KF, int NS, int EPI>
__global__ __launch_bounds__(64 * WGM * WGN)
__attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_mfma_kernel(GemmArgs p, int n_colblk, int n_rowblk) {
  using G = MfmaGeom<BM, BN, WGM, WGN, KF, NS>;
  static_assert(WGM * WGN == 4, "one wave per SIMD");
  constexpr int TM = G::TM, TN = G::TN, AT = G::AT, BT = G::BT, SF = G::SF, FPW = G::FPW;
  constexpr int NW = G::NW;
  __shared__ u32x4 lds[NS][SF][64];
  __shared__ unsigned long long kred[EPI == EPI_ARGMAX ? BM * WGN : 1];

  // Block numbering: ids 8 apart share an XCD; row blocks of one column block
  // get consecutive multiples of 8. With a K split, the slice index is the
  // slowest-varying part of the id.
  const int per_split = gridDim.x / p_ksplit(p);
  const int z = blockIdx.x / per_split;
  const int id = blockIdx.x - z * per_split;
  const int xcd = id & 7, q = id >> 3;
  const int rb = q % n_rowblk;
  const int cb = (q / n_rowblk) * 8 + xcd;
  if constexpr (EPI == EPI_STORE_F32) gemm_snapshot(p, blockIdx.x == 0);
  if (cb >= n_colblk) return;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  const int r = lane & 15, grp = lane >> 4;
  const int nck = (p.K + kKC - 1) / kKC;
  // The host guarantees K % (32 KF) == 0; slice z takes stages [s0, s0 + nst).
  const int nst_all = p.K / (32 * KF);
  const int per_slice = (nst_all + p_ksplit(p) - 1) / p_ksplit(p);
  const int s0 = z * per_slice;
  const int nst = max(0, min(per_slice, nst_all - s0));
  const int m_tiles = (p.M + 15) >> 4, n_tiles = (p.N + 15) >> 4;
  const int tile_m0 = rb * AT;
  // SwiGLU: the block's W tiles are BT/2 gate tiles then the same BT/2 up tiles.
  constexpr bool SW = EPI == EPI_SWIGLU;
  const int tile_n0 = cb * (SW ? BT / 2 : BT);

  const bf16* A = reinterpret_cast<const bf16*>(p.a[0]);
  const bf16* W = reinterpret_cast<const bf16*>(p.w);
  const bf16* W2 = reinterpret_cast<const bf16*>(p.w2);

  // Fragments this wave copies per stage: j = wave + NW * i. Stage slot j:
  // j < KF*AT: A row tile j / KF, fragment j % KF of the stage; else W tile
  // (j - KF*AT) / KF. Tiles past the matrix re-read its last tile (valid
  // memory; those rows and columns are never stored). Bases are wave-uniform.
  const bf16* src[FPW];
  int kf[FPW];
#pragma unroll
  for (int i = 0; i < FPW; ++i) {
    const int j = wave + NW * i;
    kf[i] = j % KF;
    if (j < KF * AT) {
      const int t = min(tile_m0 + j / KF, m_tiles - 1);
      src[i] = A + (int64_t)t * nck * 4 * kFRAG;
    } else {
      const int bt = (j - KF * AT) / KF;
      const bf16* base = W;
      int t = tile_n0 + bt;
      if constexpr (SW) {
        if (bt >= BT / 2) {
          base = W2;
          t = tile_n0 + bt - BT / 2;
        }
      }
      t = min(t, n_tiles - 1);
      src[i] = base + (int64_t)t * nck * 4 * kFRAG;
    }
  }

  // Stage s covers fragments KF*s .. KF*s + KF-1 of each tile's K (fragment
  // g = 4 * chunk + f sits at element g * kFRAG of the tile).
  auto issue = [&](int s, int slot) {
#pragma unroll
    for (int i = 0; i < FPW; ++i) {
      const bf16* g = src[i] + (int64_t)(KF * (s0 + s) + kf[i]) * kFRAG + lane * kEPF;
      __builtin_amdgcn_global_load_lds((gbl_ptr_t)g, (lds_ptr_t)&lds[slot][wave + NW * i][0], 16, 0,
                                       0);
    }
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // LDS index of the wave's B tile j (SwiGLU: first TN/2 gate, then up).
  auto btile = [&](int j) -> int {
    if constexpr (SW) return j < TN / 2 ? wn * (TN / 2) + j : BT / 2 + wn * (TN / 2) + j - TN / 2;
    else return wn * TN + j;
  };

  // One stage's MFMA operands in registers.
  struct Frags {
    u32x4 a[KF][TM];
    u32x4 b[KF][TN];
  };
  auto lds_read = [&](Frags& F, int slot) {
#pragma unroll
    for (int k2 = 0; k2 < KF; ++k2) {
#pragma unroll
      for (int i = 0; i < TM; ++i) F.a[k2][i] = lds[slot][(wm * TM + i) * KF + k2][lane];
#pragma unroll
      for (int j = 0; j < TN; ++j) F.b[k2][j] = lds[slot][KF * AT + btile(j) * KF + k2][lane];
    }
  };
  // The stage's MFMAs, with the next stage's LDS reads (if any) interleaved:
  // one read per MFMA_PER_READ MFMAs, so the reads' latency hides under the
  // matrix work of this wave instead of stalling it.
  constexpr int NMFMA = KF * TM * TN, NREAD = KF * (TM + TN);
  constexpr int MFMA_PER_READ = NMFMA / NREAD > 0 ? NMFMA / NREAD : 1;
  auto mma = [&](const Frags& F, Frags* next, int next_slot) {
    if (next) lds_read(*next, next_slot);
#pragma unroll
    for (int k2 = 0; k2 < KF; ++k2)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma_frag<bf16>(F.a[k2][i], F.b[k2][j], acc[i][j]);
    if (next) {
#pragma unroll
      for (int g = 0; g < NREAD; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);              // one LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, MFMA_PER_READ, 0);  // then MFMAs
      }
    }
  };

  // Ring of NS slots, all NS filled up front. Iteration s: every wave's LDS
  // reads of stage s have returned (its operands are in registers) and every
  // wave passes the barrier, so slot s % NS is free and stage s + NS is issued
  // into it; stage s + 1 has landed (each wave waited for its own loads
  // before the barrier). Stage s+1's LDS reads go out between stage s's
  // MFMAs.
#pragma unroll
  for (int st = 0; st < NS; ++st)
    if (st < nst) issue(st, st);
  if (nst >= NS) wait_loads_and_barrier<FPW * (NS - 1)>();
  else wait_loads_and_barrier<0>();
  Frags f0, f1;
  lds_read(f0, 0);
  auto step = [&](int s, Frags& cur, Frags& nxt) {
    const int slot = s % NS;
    if (s + 1 < nst) {
      // Issued so far: stages up to min(nst, s + NS) - 1, so stage s+1 has
      // landed once at most min(NS - 2, nst - 2 - s) later stages are outstanding.
      if (s + NS <= nst) wait_loads_and_barrier<FPW * (NS - 2)>();
      else wait_loads_and_barrier<0>();
      if (s + NS < nst) issue(s + NS, slot);
      mma(cur, &nxt, (s + 1) % NS);
    } else {
      mma(cur, nullptr, 0);
    }
  };
  int s = 0;
  for (; s + 1 < nst; s += 2) {
    step(s, f0, f1);
    step(s + 1, f1, f0);
  }
  if (s < nst) step(s, f0, f1);
  __syncthreads();

  // Epilogue. Lane (r, grp) of tile (i, j) holds rows 4*grp + e of column r.
  const int row0 = tile_m0 * 16 + wm * (TM * 16);
  if constexpr (EPI == EPI_STORE_F32 || EPI == EPI_RESID) {
    if (p_ksplit(p) > 1) {
      // K slice z: fp32 partial tile, summed in slice order by splitk_reduce_kernel.
      float* part = p.part + (int64_t)z * p.M * p.N;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int n = (tile_n0 + wn * TN + j) * 16 + r;
          if (n >= p.N) continue;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int m = row0 + 16 * i + 4 * grp + e;
            if (m < p.M) part[(int64_t)m * p.N + n] = acc[i][j][e];
          }
        }
      return;
    }
  }
  if constexpr (EPI == EPI_ARGMAX) {
    // Per row: max over this wave's columns, then over the WGN waves via LDS.
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = row0 + 16 * i + 4 * grp + e;
        unsigned long long key = 0ull;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int n = (tile_n0 + wn * TN + j) * 16 + r;
          if (n < p.N) {
            if (p.logits && m < p.M)
              p.logits[(int64_t)m * p.logits_stride + p.col0 + n] = acc[i][j][e];
            const unsigned long long k = argmax_key(acc[i][j][e], (unsigned)(p.col0 + n));
            key = k > key ? k : key;
          }
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
          const unsigned long long other = __shfl_xor(key, o);
          key = other > key ? other : key;
        }
        if (r == 0) kred[(wm * TM * 16 + 16 * i + 4 * grp + e) * WGN + wn] = key;
      }
    }
    __syncthreads();
    for (int row = threadIdx.x; row < BM; row += 64 * NW) {
      const int m = tile_m0 * 16 + row;
      if (m < p.M) {
        unsigned long long best = 0ull;
#pragma unroll
        for (int w = 0; w < WGN; ++w) {
          const unsigned long long k = kred[row * WGN + w];
          best = k > best ? k : best;
        }
        p.amax[(int64_t)m * p.amax_stride + p.amax_col0 + cb] = best;
      }
    }
  } else if constexpr (SW) {
    bf16* out = reinterpret_cast<bf16*>(p.out);
    const int out_nck = (p.N + kKC - 1) / kKC;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN / 2; ++j) {
        const int n = (tile_n0 + wn * (TN / 2) + j) * 16 + r;
        if (n >= p.N) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = row0 + 16 * i + 4 * grp + e;
          if (m < p.M) {
            const float gt = acc[i][j][e];
            const float silu = gt / (1.0f + __expf(-gt));
            out[tiled_index<bf16>(m, n, out_nck)] = (bf16)(silu * acc[i][j + TN / 2][e]);
          }
        }
      }
  } else if constexpr (EPI == EPI_STORE_F32) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = (tile_n0 + wn * TN + j) * 16 + r;
        if (n >= p.N) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = row0 + 16 * i + 4 * grp + e;
          if (m < p.M) reinterpret_cast<float*>(p.out)[(int64_t)m * p.out_stride + n] = acc[i][j][e];
        }
      }
  } else {
    resid_add_tiles<TM, TN>(p, acc, row0, (tile_n0 + wn * TN) * 16 + r, grp);
  }
}

// Eight waves (two per SIMD) over a 256-row block, k = 32 per stage in an
// NS-slot LDS ring, and everything a stage needs besides its MFMAs hidden
// inside them. The block's data for one stage is one 1 KB fragment per
// 16-row tile of A and of W: (BM + BN) / 16 fragments, split over the waves.
// Iteration s of the loop:
//   * wait until stage s+1 has landed and every wave holds stage s in
//     registers (vmcnt + lgkmcnt, then a barrier), so the slot of stage s is
//     free;
//   * run stage s's MFMAs from registers in program order, fenced in groups
//     of MPR: after each group one LDS read of stage s+1's operands (into the
//     second register set), and after the first groups this wave's loads of
//     stage s+NS into the freed slot.
// The loads go out one at a time between MFMAs instead of all waves queueing
// theirs at the same moment after the barrier, which stalled the issuing
// waves (measured: +10-25% at 480-2048 rows); the LDS reads of the next
// stage overlap the current MFMAs. Every iteration issues a stage (past the
// end: the slice's last stage again, into a slot nobody reads any more), so
// the wait count is the same in every iteration and the loop has no branches
// (branches in the loop made the register allocator spill the accumulators).
// LDS holds nothing but the ring during the loop: a second LDS array made the
// compiler wait for every outstanding global->LDS load before each LDS read.
template <int BM, int BN, int WGM, int WGN, int NS, int EPI>
__global__ __launch_bounds__(64 * WGM * WGN)
__attribute__((amdgpu_waves_per_eu(WGM * WGN / 4, WGM * WGN / 4)))
void gemm_pipe_kernel(GemmArgs p, int n_colblk, int n_rowblk) {
  constexpr int NW = WGM * WGN;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int TM = WM / 16, TN = WN / 16;
  constexpr int AT = BM / 16, BT = BN / 16;
  constexpr int SF = AT + BT;             // fragments per stage
  constexpr int FPW = (SF + NW - 1) / NW; // loads per wave per stage (the last may be idle)
  constexpr bool SW = EPI == EPI_SWIGLU;
  static_assert(NS >= 3, "a slot being read, one arriving, one being filled");
  static_assert(!SW || TN % 2 == 0, "SwiGLU pairs gate and up tiles");
  __shared__ u32x4 lds[NS][SF][64];

  const int per_split = gridDim.x / p_ksplit(p);
  const int z = blockIdx.x / per_split;
  const int id = blockIdx.x - z * per_split;
  const int xcd = id & 7, q = id >> 3;
  const int rb = q % n_rowblk;
  const int cb = (q / n_rowblk) * 8 + xcd;
  if constexpr (EPI == EPI_STORE_F32) gemm_snapshot(p, blockIdx.x == 0);
  if (cb >= n_colblk) return;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  const int r = lane & 15, grp = lane >> 4;
  const int nck = (p.K + kKC - 1) / kKC;
  // The host guarantees K % 64 == 0 and an even number of stages per slice.
  const int nst_all = p.K / 32;
  const int nst = nst_all / p_ksplit(p);
  const int s0 = z * nst;
  const int m_tiles = (p.M + 15) >> 4, n_tiles = (p.N + 15) >> 4;
  const int tile_m0 = rb * AT;
  const int tile_n0 = cb * (SW ? BT / 2 : BT);

  const bf16* A = reinterpret_cast<const bf16*>(p.a[0]);
  const bf16* W = reinterpret_cast<const bf16*>(p.w);
  const bf16* W2 = reinterpret_cast<const bf16*>(p.w2);

  // Fragment j = wave + NW * i of a stage: j < AT: A row tile j, else W tile
  // j - AT (SwiGLU: BT/2 gate tiles, then the same BT/2 up tiles). Tiles past
  // the matrix re-read its last tile (valid memory, never stored).
  const bf16* src[FPW];
#pragma unroll
  for (int i = 0; i < FPW; ++i) {
    const int j = min(wave + NW * i, SF - 1);
    const bf16* base;
    int t;
    if (j < AT) {
      base = A;
      t = min(tile_m0 + j, m_tiles - 1);
    } else {
      const int bt = j - AT;
      base = W;
      t = tile_n0 + bt;
      if constexpr (SW) {
        if (bt >= BT / 2) {
          base = W2;
          t = tile_n0 + bt - BT / 2;
        }
      }
      t = min(t, n_tiles - 1);
    }
    src[i] = base + ((int64_t)t * nck * 4 + s0) * kFRAG + lane * kEPF;
  }
  // When the stage's fragments do not split evenly, waves >= SF % NW have one
  // load fewer (the last), and wait for correspondingly fewer.
  constexpr bool EVEN = SF % NW == 0;
  const bool full = EVEN || wave < SF % NW;  // wave-uniform
  auto load = [&](int i, int st, int slot) {
    if (EVEN || i < FPW - 1 || full)
      __builtin_amdgcn_global_load_lds((gbl_ptr_t)(src[i] + (int64_t)st * kFRAG),
                                       (lds_ptr_t)&lds[slot][wave + NW * i][0], 16, 0, 0);
  };
  // Stage s+1 landed: at most `later` stages of this wave's loads outstanding.
  auto wait_stage = [&](auto later) {
    constexpr int L = decltype(later)::value;
    if (full) wait_loads_and_barrier<FPW * L>();
    else wait_loads_and_barrier<(FPW - 1) * L>();
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // LDS index of the wave's B tile j (SwiGLU: first TN/2 gate, then up).
  auto btile = [&](int j) -> int {
    if constexpr (SW) return j < TN / 2 ? wn * (TN / 2) + j : BT / 2 + wn * (TN / 2) + j - TN / 2;
    else return wn * TN + j;
  };
  struct Ops {
    u32x4 a[TM];
    u32x4 b[TN];
  };
  auto read_one = [&](Ops& O, int slot, int k) {
    if (k < TM) O.a[k] = lds[slot][wm * TM + k][lane];
    else O.b[k - TM] = lds[slot][AT + btile(k - TM)][lane];
  };
  constexpr int NMFMA = TM * TN, NREAD = TM + TN;
  constexpr int MPR = NMFMA / NREAD > 0 ? NMFMA / NREAD : 1;
  static_assert(NREAD >= FPW, "one load per read group");
  auto compute = [&](const Ops& C) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = mfma_frag<bf16>(C.a[i], C.b[j], acc[i][j]);
  };
  // Groups of MPR MFMAs, each with one LDS read of the next stage (and, in
  // the first FPW groups, one load), fenced from the next group; the
  // compiler places each read ahead of its group's MFMAs.
  auto stage = [&](int s, const Ops& C, Ops& N) {
    wait_stage(std::integral_constant<int, NS - 2>());
    const int ist = min(s + NS, nst - 1), islot = s % NS, nslot = (s + 1) % NS;
    __builtin_amdgcn_sched_barrier(0);
    int rd = 0;
#pragma unroll
    for (int t = 0; t < NMFMA; ++t) {
      acc[t / TN][t % TN] = mfma_frag<bf16>(C.a[t / TN], C.b[t % TN], acc[t / TN][t % TN]);
      if ((t + 1) % MPR == 0 && rd < NREAD) {
        read_one(N, nslot, rd);
        if (rd < FPW) load(rd, ist, islot);
        ++rd;
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

#pragma unroll
  for (int st = 0; st < NS; ++st)
#pragma unroll
    for (int i = 0; i < FPW; ++i) load(i, min(st, nst - 1), st);
  wait_stage(std::integral_constant<int, NS - 1>());
  Ops r0, r1;
#pragma unroll
  for (int k = 0; k < NREAD; ++k) read_one(r0, 0, k);
  for (int s = 0; s < nst - 2; s += 2) {
    stage(s, r0, r1);
    stage(s + 1, r1, r0);
  }
  stage(nst - 2, r0, r1);
  compute(r1);
  __syncthreads();

  // Epilogue. Lane (r, grp) of tile (i, j) holds rows 4*grp + e of column r.
  const int row0 = tile_m0 * 16 + wm * (TM * 16);
  if constexpr (EPI == EPI_STORE_F32 || EPI == EPI_RESID) {
    if (p_ksplit(p) > 1) {
      // K slice z: fp32 partial tile, summed in slice order by splitk_reduce_kernel.
      float* part = p.part + (int64_t)z * p.M * p.N;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int n = (tile_n0 + wn * TN + j) * 16 + r;
          if (n >= p.N) continue;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int m = row0 + 16 * i + 4 * grp + e;
            if (m < p.M) part[(int64_t)m * p.N + n] = acc[i][j][e];
          }
        }
      return;
    }
  }
  if constexpr (EPI == EPI_ARGMAX) {
    // The ring is free after the loop: it holds the per-wave row keys.
    static_assert((int64_t)BM * WGN * 8 <= (int64_t)NS * SF * 64 * 16, "key scratch");
    unsigned long long* kred = reinterpret_cast<unsigned long long*>(&lds[0][0][0]);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = row0 + 16 * i + 4 * grp + e;
        unsigned long long key = 0ull;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int n = (tile_n0 + wn * TN + j) * 16 + r;
          if (n < p.N) {
            if (p.logits && m < p.M)
              p.logits[(int64_t)m * p.logits_stride + p.col0 + n] = acc[i][j][e];
            const unsigned long long k = argmax_key(acc[i][j][e], (unsigned)(p.col0 + n));
            key = k > key ? k : key;
          }
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
          const unsigned long long other = __shfl_xor(key, o);
          key = other > key ? other : key;
        }
        if (r == 0) kred[(wm * TM * 16 + 16 * i + 4 * grp + e) * WGN + wn] = key;
      }
    }
    __syncthreads();
    for (int row = threadIdx.x; row < BM; row += 64 * NW) {
      const int m = tile_m0 * 16 + row;
      if (m < p.M) {
        unsigned long long best = 0ull;
#pragma unroll
        for (int w = 0; w < WGN; ++w) {
          const unsigned long long k = kred[row * WGN + w];
          best = k > best ? k : best;
        }
        p.amax[(int64_t)m * p.amax_stride + p.amax_col0 + cb] = best;
      }
    }
  } else if constexpr (SW) {
    bf16* out = reinterpret_cast<bf16*>(p.out);
    const int out_nck = (p.N + kKC - 1) / kKC;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN / 2; ++j) {
        const int n = (tile_n0 + wn * (TN / 2) + j) * 16 + r;
        if (n >= p.N) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = row0 + 16 * i + 4 * grp + e;
          if (m < p.M) {
            const float gt = acc[i][j][e];
            const float silu = gt / (1.0f + __expf(-gt));
            out[tiled_index<bf16>(m, n, out_nck)] = (bf16)(silu * acc[i][j + TN / 2][e]);
          }
        }
      }
  } else if constexpr (EPI == EPI_STORE_F32) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = (tile_n0 + wn * TN + j) * 16 + r;
        if (n >= p.N) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = row0 + 16 * i + 4 * grp + e;
          if (m < p.M) reinterpret_cast<float*>(p.out)[(int64_t)m * p.out_stride + n] = acc[i][j][e];
        }
      }
  } else {
    resid_add_tiles<TM, TN>(p, acc, row0, (tile_n0 + wn * TN) * 16 + r, grp);
  }
}

// Column blocks per launch for an epilogue: SwiGLU blocks hold BN/2 output
// columns (gate and up tiles side by side).
static int mfma_colblocks(int epi, int N, int BN) {
  const int cols = epi == EPI_SWIGLU ? BN / 2 : BN;
  return (N + cols - 1) / cols;
}

// Block shapes: 256x256 (8 waves of 128x64, pipelined), 256x192 (8 waves of
// 64x96, pipelined), 256x128 and 128x256 (8 waves of 64x64, pipelined),
// 128x128 (4 waves of 64x64), 128x96 (4 waves of 64x48). Bigger blocks read
// fewer operand bytes per flop; smaller ones fill the 256 CUs at fewer rows
// or columns. Each shape is costed by what one workgroup takes on MI355X
// with every CU busy (bf16, random data, weights streamed from HBM; timed at
// 261-512 rows): `tflops` per CU once the ring is full, plus `fixed_us` per
// workgroup for filling the ring, the epilogue and its stores (a 128x128
// workgroup over K = 4096 on 256 CUs: 21 + 6.6 us). Fewer busy CUs clock
// higher, ~35% more per CU when almost all are idle.
struct MfmaShape {
  int bm, bn;
  bool pipe;
  double tflops;
  double fixed_us;
};
static constexpr int kNShapes = 7;
static const MfmaShape kShapes[kNShapes] = {
    {256, 256, true, 4.96, 6.8},  {256, 192, true, 4.84, 6.5}, {256, 128, true, 4.6, 6.1},
    {128, 256, true, 4.75, 8.3},  {128, 128, false, 3.18, 6.6}, {128, 96, false, 3.45, 5.0},
    {96, 256, true, 4.3, 8.3}};

// Whether a shape can take K slices of ks: fp32-store / residual epilogues
// only (slices write fp32 partials that a reduce kernel sums in order). The
// pipelined kernel needs an even number of k = 32 stages per slice, and at
// least 32 of them (shorter slices spend more on filling the ring and
// storing partials than they gain: 256x256 blocks over 16 stages ran no faster
// than 128x128 ones over 32); the 4-wave one >= 8 stages of k = 64.
static bool ksplit_ok(const MfmaShape& sh, int epi, int K, int ks) {
  if (ks == 1) return true;
  if (epi != EPI_STORE_F32 && epi != EPI_RESID) return false;
  if (sh.pipe) return (K / 32) % (2 * ks) == 0 && K / 32 / ks >= 32;
  return (K / 64) % ks == 0 && K / 64 / ks >= 8;
}

// Estimated time (us) of one launch: rounds of up to 256 workgroups, each
// block of bm x bn x K/ks at the shape's rate per CU (raised when the round
// leaves CUs idle) plus its fixed cost, plus, with K slices, the store of its
// fp32 partial block at ~60 GB/s per CU; 256-row blocks that are more than a
// quarter padding ran ~15% slower than their flops say (136 rows: 56.6 us
// against 49.5 for two 128-row blocks); then the output traffic at ~5 TB/s:
// without slices the residual's read-modify-write (latency-bound at the end
// of a block: counted 3x) or the fp32 store; with slices the reduce kernel,
// whose cost per 2^21 output elements was measured as 8.0 + 0.95 ks us with
// the residual add and RMSNorm (2, 4, 8 slices: 9.9, 11.7, 15.5 us) and
// 1.0 + 1.6 ks us for a plain sum (4.7, 9.9, 16.6 us at 1.5 x that size;
// rounded up: the slices' partial stores also slow their own GEMM).
static double mfma_time_us(const MfmaShape& sh, int epi, int M, int N, int K, int ks) {
  const long long wgs = (long long)((M + sh.bm - 1) / sh.bm) * mfma_colblocks(epi, N, sh.bn) * ks;
  const double block_mflop = 2.0 * sh.bm * sh.bn * ((double)K / ks) * 1e-6;
  const int rows = ((M + sh.bm - 1) / sh.bm) * sh.bm;
  const double pad_penalty = (sh.bm == 256 && 4 * (rows - M) > rows) ? 1.15 : 1.0;
  const double part_us = ks > 1 ? (double)sh.bm * sh.bn * 4 / 60e3 : 0.0;
  double t = 0;
  for (long long left = wgs; left > 0; left -= 256) {
    const double busy = (double)(left < 256 ? left : 256);
    t += pad_penalty * block_mflop / (sh.tflops * (1.0 + 0.35 * (1.0 - busy / 256.0))) +
         sh.fixed_us + part_us;
  }
  const double out_mb = (double)M * N * 4 * 1e-6;
  const double units = (double)M * N / (double)(1 << 21);
  if (ks > 1) t += (epi == EPI_RESID ? 8.0 + 0.95 * ks : 1.0 + 1.6 * ks) * units;
  else t += (epi == EPI_RESID ? 3.0 : epi == EPI_STORE_F32 ? 1.0 : 0.0) * out_mb / 5.0;
  return t;
}

struct MfmaPlan {
  int shape, ksplit;
};
// The shape and K split with the least estimated time. SwiGLU needs an even
// number of column tiles per wave (not 128x96); the LM-head argmax keeps
// square blocks. Ties go to the earlier shape and fewer slices.
static MfmaPlan mfma_plan(int epi, int M, int N, int K) {
  MfmaPlan best{0, 1};
  double best_t = 1e300;
  for (int i = 0; i < kNShapes; ++i) {
    const MfmaShape& sh = kShapes[i];
    if (epi == EPI_SWIGLU && sh.bn == 96) continue;
    // 96-row blocks (waves of 48x64) only for stores and residual adds whose
    // rows they cover with less padding than 128-row blocks (261 rows: 288
    // computed instead of 384).
    if (sh.bm == 96 && (epi == EPI_SWIGLU || epi == EPI_ARGMAX ||
                        (M + 95) / 96 * 96 >= (M + 127) / 128 * 128))
      continue;
    if (epi == EPI_ARGMAX && sh.bm != sh.bn) continue;
    if (sh.pipe && (K / 32) % 2) continue;
    for (int ks = 1; ks <= kMfmaMaxSplit; ks *= 2) {
      if (ks > 1 && (int64_t)M * N > kMfmaSplitMaxElems) break;
      if (!ksplit_ok(sh, epi, K, ks)) continue;
      const double t = mfma_time_us(sh, epi, M, N, K, ks);
      if (t < best_t * 0.999) {
        best_t = t;
        best = MfmaPlan{i, ks};
      }
    }
  }
  return best;
}

int mfma_gemm_colblocks(int epi, int M, int N, int K) {
  return mfma_colblocks(epi, N, kShapes[mfma_plan(epi, M, N, K).shape].bn);
}

// The LM head on 256x256 blocks: when its last round of 256 workgroups
// would be less than three quarters full (batch 32: 1188 workgroups, 4.64
// rounds), the columns of the full rounds stay on 256x256 blocks and the rest
// runs as a second launch of 256x192 blocks that fits one round (218
// workgroups at three quarters of the work each, instead of 164 full ones):
// the last round then takes ~0.75 of a round's time. Returns the column
// blocks of the first launch (0: no split) and, in *tail, of the second.
static int lm_head_split(int M, int N, int K, int* tail) {
  *tail = 0;
  const MfmaPlan pl = mfma_plan(EPI_ARGMAX, M, N, K);
  if (pl.shape != 0) return 0;
  const int rb = (M + 255) / 256, cb = mfma_colblocks(EPI_ARGMAX, N, 256);
  const int wgs = rb * cb, rounds = wgs / 256, last = wgs - rounds * 256;
  if (rounds < 1 || last == 0 || 4 * last >= 3 * 256) return 0;
  const int cb_main = rounds * 256 / rb;
  const int n_tail = N - cb_main * 256;
  const int cb_tail = mfma_colblocks(EPI_ARGMAX, n_tail, 192);
  if (n_tail <= 0 || cb_tail * rb > 256) return 0;
  *tail = cb_tail;
  return cb_main;
}

int mfma_argmax_keys(int M, int N, int K) {
  int tail = 0;
  const int main = lm_head_split(M, N, K, &tail);
  return main > 0 ? main + tail : mfma_gemm_colblocks(EPI_ARGMAX, M, N, K);
}

int mfma_gemm_ksplit(int epi, int M, int N, int K) { return mfma_plan(epi, M, N, K).ksplit; }

// Sum of the K-slice partials in slice order, then the projection's epilogue:
// out = sum (EPI_STORE_F32) or resid += sum (EPI_RESID). Four columns per thread.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int ks,
                                                            int M, int N, float* out,
                                                            int64_t out_stride, int resid) {
  const int64_t n4 = (int64_t)M * N / 4;
  const int64_t MN = (int64_t)M * N;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * blockDim.x) {
    float4 acc = reinterpret_cast<const float4*>(part)[i];
    for (int z = 1; z < ks; ++z) {
      const float4 v = reinterpret_cast<const float4*>(part + z * MN)[i];
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    const int64_t e = 4 * i;
    const int m = (int)(e / N), n = (int)(e % N);
    float4* dst = reinterpret_cast<float4*>(out + (int64_t)m * out_stride + n);
    if (resid) {
      const float4 x = *dst;
      acc.x += x.x;
      acc.y += x.y;
      acc.z += x.z;
      acc.w += x.w;
    }
    *dst = acc;
  }
}

// Sums the K slices' partials into the projection's output (launched after
// the GEMM on the same stream), with the RMSNorm of the updated rows when the
// caller asked for it.
static hipError_t launch_splitk_reduce(int epi, const GemmArgs& a, hipStream_t st) {
  if ((epi == EPI_RESID || epi == EPI_STORE_F32) && a.norm_w)
    return launch_splitk_reduce_norm(a.part, a.ksplit, a.M, a.N, a.resid, a.out_stride, a.norm_w,
                                     a.norm_out, a.norm_nck, a.norm_eps, epi == EPI_RESID,
                                     epi == EPI_RESID ? a.norm_block : 0, st);
  float* dst = epi == EPI_RESID ? a.resid : reinterpret_cast<float*>(a.out);
  const int64_t n4 = (int64_t)a.M * a.N / 4;
  const int blocks = (int)std::min<int64_t>((n4 + 255) / 256, 4096);
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3(blocks), dim3(256), 0, st, a.part, a.ksplit, a.M,
                     a.N, dst, a.out_stride, epi == EPI_RESID ? 1 : 0);
  return hipGetLastError();
}

// The K split the plan asks for, if the caller's partial buffer and the
// output layout allow it (else 1).
static int usable_ksplit(int epi, const GemmArgs& a) {
  if (epi != EPI_STORE_F32 && epi != EPI_RESID) return 1;
  const int ks = mfma_gemm_ksplit(epi, a.M, a.N, a.K);
  if (ks > 1 && a.part && a.part_elems >= (int64_t)ks * a.M * a.N && a.N % 4 == 0 &&
      a.out_stride % 4 == 0)
    return ks;
  return 1;
}

int gemm_store_slices(int dtype, const GemmArgs& a) {
  if (!gemm_uses_mfma(dtype, a.M, a.K, a.a_tiled != 0, EPI_STORE_F32)) return 1;
  return usable_ksplit(EPI_STORE_F32, a);
}

bool gemm_fuses_norm(int dtype, const GemmArgs& a, int epi) {
  return (epi == EPI_RESID || epi == EPI_STORE_F32) &&
         gemm_uses_mfma(dtype, a.M, a.K, a.a_tiled != 0, epi) && usable_ksplit(epi, a) > 1 &&
         a.N <= 8192;
}

template <int BM, int BN, int WGM, int WGN, int KF, int NS, int EPI>
static hipError_t launch_mfma_t(const GemmArgs& a0, hipStream_t st) {
  GemmArgs a = a0;
  a.ksplit = usable_ksplit(EPI, a);
  const int n_colblk = mfma_colblocks(EPI, a.N, BN);
  const int n_rowblk = (a.M + BM - 1) / BM;
  const int groups = (n_colblk + 7) / 8;
  const dim3 grid(groups * 8 * n_rowblk * a.ksplit), block(64 * WGM * WGN);
  hipLaunchKernelGGL((gemm_mfma_kernel<BM, BN, WGM, WGN, KF, NS, EPI>), grid, block, 0, st,
                     a, n_colblk, n_rowblk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.ksplit == 1 || (EPI == EPI_STORE_F32 && a.defer_reduce)) return e;
  return launch_splitk_reduce(EPI, a, st);
}

template <int BM, int BN, int WGM, int WGN, int NS, int EPI>
static hipError_t launch_pipe_t(const GemmArgs& a0, hipStream_t st) {
  GemmArgs a = a0;
  a.ksplit = usable_ksplit(EPI, a);
  if ((a.K / 32) % (2 * a.ksplit)) return hipErrorInvalidValue;
  const int n_colblk = mfma_colblocks(EPI, a.N, BN);
  const int n_rowblk = (a.M + BM - 1) / BM;
  const int groups = (n_colblk + 7) / 8;
  const dim3 grid(groups * 8 * n_rowblk * a.ksplit), block(64 * WGM * WGN);
  hipLaunchKernelGGL((gemm_pipe_kernel<BM, BN, WGM, WGN, NS, EPI>), grid, block, 0, st, a,
                     n_colblk, n_rowblk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.ksplit == 1 || (EPI == EPI_STORE_F32 && a.defer_reduce)) return e;
  return launch_splitk_reduce(EPI, a, st);
}

template <int EPI>
static hipError_t launch_mfma_epi(const GemmArgs& a, hipStream_t st) {
  // Pipelined shapes: 4 ring slots of k = 32 for the LM head (128 KB; its
  // weights stream from HBM once), 3 for the others (96 / 84 KB); the 4-wave
  // shapes keep stages of k = 64 in 4 slots (32 / 28 KB each).
  if constexpr (EPI == EPI_ARGMAX) {
    int cb_tail = 0;
    const int cb_main = lm_head_split(a.M, a.N, a.K, &cb_tail);
    if (cb_main > 0) {
      GemmArgs m = a, t = a;
      m.N = cb_main * 256;
      hipError_t e = launch_pipe_t<256, 256, 2, 4, 4, EPI>(m, st);
      if (e != hipSuccess) return e;
      t.N = a.N - m.N;
      t.w = reinterpret_cast<const bf16*>(a.w) + (int64_t)(m.N / 16) * ((a.K + kKC - 1) / kKC) * 4 * kFRAG;
      t.col0 = a.col0 + m.N;
      t.amax_col0 = a.amax_col0 + cb_main;
      return launch_pipe_t<256, 192, 4, 2, 4, EPI>(t, st);
    }
  }
  // The 64x64-wave pipelined shapes keep 4 ring slots of k = 32 (96 KB).
  switch (mfma_plan(EPI, a.M, a.N, a.K).shape) {
    case 0:
      if constexpr (EPI == EPI_ARGMAX) return launch_pipe_t<256, 256, 2, 4, 4, EPI>(a, st);
      else return launch_pipe_t<256, 256, 2, 4, 3, EPI>(a, st);
    case 1:
      if constexpr (EPI == EPI_ARGMAX) return hipErrorInvalidValue;
      else return launch_pipe_t<256, 192, 4, 2, 3, EPI>(a, st);
    case 2:
      if constexpr (EPI == EPI_ARGMAX) return hipErrorInvalidValue;
      else return launch_pipe_t<256, 128, 4, 2, 4, EPI>(a, st);
    case 3:
      if constexpr (EPI == EPI_ARGMAX) return hipErrorInvalidValue;
      else return launch_pipe_t<128, 256, 2, 4, 4, EPI>(a, st);
    case 4: return launch_mfma_t<128, 128, 2, 2, 2, 4, EPI>(a, st);
    case 6:
      if constexpr (EPI == EPI_ARGMAX || EPI == EPI_SWIGLU) return hipErrorInvalidValue;
      else return launch_pipe_t<96, 256, 2, 4, 4, EPI>(a, st);
    default:
      if constexpr (EPI == EPI_ARGMAX || EPI == EPI_SWIGLU) return hipErrorInvalidValue;
      else return launch_mfma_t<128, 96, 2, 2, 2, 4, EPI>(a, st);
  }
}

hipError_t launch_gemm_mfma(int epi, const GemmArgs& a, hipStream_t st) {
  if (a.M <= 0 || a.N <= 0 || a.K <= 0) return hipSuccess;
  if (!a.a_tiled || a.K % 64) return hipErrorInvalidValue;
  switch (epi) {
    case EPI_STORE_F32: return launch_mfma_epi<EPI_STORE_F32>(a, st);
    case EPI_RESID: return launch_mfma_epi<EPI_RESID>(a, st);
    case EPI_SWIGLU: return launch_mfma_epi<EPI_SWIGLU>(a, st);
    default: return launch_mfma_epi<EPI_ARGMAX>(a, st);
  }
}

}  // namespace dflash
