// Host-side launch interfaces shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dflash.h"

namespace dflash {

constexpr int kMaxASeg = 8;    // K-segments of a row-major GEMM A operand (fused target features)
constexpr int kKeyBlock = 32;  // V cache position block
constexpr int kMaxLayers = 16;

enum Epilogue : int {
  EPI_STORE_F32 = 0,  // out (fp32) = acc
  EPI_RESID = 1,      // resid (fp32) += acc
  EPI_SWIGLU = 2,     // out (model dtype, tiled) = SiLU(acc_gate) * acc_up
  EPI_ARGMAX = 3,     // per-row (max, argmax) over the tile -> partial keys; optional fp32 logits
};

// Chunk width (elements) and chunk count of the tiled layout for a dtype.
inline int tiled_kc(int dtype) { return dtype == DFLASH_BF16 ? 128 : 64; }
inline int tiled_nck(int dtype, int K) { return (K + tiled_kc(dtype) - 1) / tiled_kc(dtype); }
// Bytes of a tiled [rows, K] matrix (rows padded to 16, k to the chunk).
inline size_t tiled_bytes(int dtype, int64_t rows, int K) {
  return (size_t)((rows + 15) / 16) * 16 * (size_t)tiled_nck(dtype, K) * tiled_kc(dtype) *
         (dtype == DFLASH_BF16 ? 2 : 4);
}

// Y[M, N] = A[M, K] · W[N, K]^T with a fused epilogue.
//  W (and w2, the up matrix of EPI_SWIGLU): tiled [N, K] (layout in common.h).
//  A: a_tiled = 1: a[0] is a tiled [M, K] matrix (activations the library
//     wrote itself); a_tiled = 0: row-major, row m, column k at
//     a[k / a_seg_k] + m * a_stride + k % a_seg_k (caller inputs; a_nseg > 1
//     places several [M, a_seg_k] matrices side by side along k).
struct GemmArgs {
  const void* a[kMaxASeg];
  int64_t a_stride;
  int a_seg_k;
  int a_nseg;
  int a_tiled;
  const void* w;
  const void* w2;
  int M, N, K;
  int k_per_wave;                 // K range per wave (multiple of the chunk)
  void* out;                      // EPI_STORE_F32: fp32 [M, out_stride]; EPI_SWIGLU: tiled [M, N]
  int64_t out_stride;
  float* resid;                   // EPI_RESID: fp32 [M, out_stride]
  unsigned long long* amax;       // EPI_ARGMAX: [M][n_tiles] partial keys
  int64_t amax_stride;
  float* logits;                  // EPI_ARGMAX, optional
  int64_t logits_stride;
  int col0;                       // EPI_ARGMAX: global column of this launch's column 0 (key
                                  // indices and logits columns are offset by it)
  int amax_col0;                  // EPI_ARGMAX: first key column of this launch in amax rows
  // Split-K scratch of the MFMA kernel (EPI_STORE_F32 / EPI_RESID only):
  // fp32 [ksplit][M][N], part_elems floats available; nullptr: never split.
  float* part;
  int64_t part_elems;
  int ksplit;                     // K slices of an MFMA launch (set by its launcher)
  int defer_reduce;               // EPI_STORE_F32: leave the K slices' partials for the
                                  // consumer to sum (gemm_store_slices of them), no reduce
  // EPI_RESID on the MFMA path with K slices (gemm_fuses_norm): the reduce of
  // the slices also writes RMSNorm(resid row; norm_w) to norm_out, tiled bf16
  // with norm_nck chunks per row. EPI_STORE_F32 likewise: the reduce writes
  // only RMSNorm(sum row; norm_w) to norm_out (row-major bf16, row stride N,
  // when norm_nck is 0), not out. Ignored (nullptr) otherwise.
  const void* norm_w;
  void* norm_out;
  int norm_nck;
  float norm_eps;
  int norm_block;                 // > 0 (EPI_RESID): residual row m is normalised only when
                                  // m % norm_block != 0, into norm_out row
                                  // (m / norm_block) * (norm_block - 1) + m % norm_block - 1
  // Weight-streaming path (bf16), the next RMSNorm deferred to its consumer:
  // an EPI_RESID projection with sq_out also writes bf16(x_new * norm_w)
  // tiled to norm_out and, for every 16-column tile j < T = ceil(N / 16) of
  // its output and row m, the sum of x_new^2 over the tile to
  // sq_out[m * T4 + j] (T4 = T rounded up to a multiple of 4; entries T..T4-1
  // unused); a projection with sq_in (its A operand such a norm_out) scales
  // output row m by 1 / sqrt(sum over j < T of sq_in[m * T4 + j] / sq_d +
  // norm_eps), T from sq_d. Unused: nullptr.
  float* sq_out;
  const float* sq_in;
  int sq_d;
  // EPI_STORE_F32 only: workgroup 0 of the projection copies snap_n int32
  // values from snap_src to snap_dst before anything else (a context-K/V
  // append snapshots ctx_len this way, so its scatter kernel reads positions
  // from the copy and may update ctx_len itself). Unused: snap_dst == nullptr.
  const int32_t* snap_src;
  int32_t* snap_dst;
  int snap_n;
};

// The snapshot of GemmArgs::snap_*, made by the workgroup whose flat index is 0.
__device__ __forceinline__ void gemm_snapshot(const GemmArgs& p, bool first_wg) {
  if (p.snap_dst && first_wg)
    for (int i = threadIdx.x; i < p.snap_n; i += blockDim.x) p.snap_dst[i] = p.snap_src[i];
}

// Launch geometry of one weight-streaming GEMM (also used to size LM-head partials).
struct GemmPlan {
  int mt, nt;           // 16-row m-tiles and 16-column n-tiles per workgroup
  int grid_x, grid_y;
  int ksplit;           // waves per workgroup, each taking k_per_wave of K
  int k_per_wave;
  size_t lds;
};
// a_seg_k: width of each A segment when A is several matrices side by side, else 0.
GemmPlan plan_gemm(int dtype, int epi, int M, int N, int K, int a_seg_k);
hipError_t launch_gemm(int dtype, int epi, const GemmArgs& args, hipStream_t st);

// Projections of at least kMfmaMinRows tiled bf16 rows with K a multiple of
// 64 run on the MFMA-bound LDS-tiled kernel (gemm_mfma.hip), the others on
// the weight-streaming one. From 64 rows the MFMA kernel (128-row blocks, K
// split) beat the weight stream on every per-layer projection (measured at
// 64 and 96 rows: QKV 23 -> 18 us, down 36 -> 30, gate/up 50 -> 45, O even);
// the LM head, whose 256-row blocks would mostly compute padding, switches
// at 128.
constexpr int kMfmaMinRows = 64;
constexpr int kMfmaMinRowsArgmax = 128;
inline bool gemm_uses_mfma(int dtype, int M, int K, bool a_tiled, int epi = EPI_STORE_F32) {
  return dtype == DFLASH_BF16 && a_tiled && K % 64 == 0 &&
         M >= (epi == EPI_ARGMAX ? kMfmaMinRowsArgmax : kMfmaMinRows);
}
hipError_t launch_gemm_mfma(int epi, const GemmArgs& a, hipStream_t st);
// K splits of the MFMA path: at most kMfmaMaxSplit slices, and only for
// outputs of at most kMfmaSplitMaxElems elements (larger ones fill the chip
// without), so the partials of any row count up to M never exceed
// kMfmaMaxSplit * min(M * N, kMfmaSplitMaxElems) floats.
constexpr int kMfmaMaxSplit = 8;
constexpr int64_t kMfmaSplitMaxElems = (int64_t)1 << 22;
int mfma_gemm_colblocks(int epi, int M, int N, int K);
// Keys per row the MFMA LM-head projection writes (its column blocks, over
// both launches when its last columns run as a second launch).
int mfma_argmax_keys(int M, int N, int K);
// K slices the MFMA kernel splits a projection into (1 = no split); the
// partial buffer it then needs is ksplit * M * N floats.
int mfma_gemm_ksplit(int epi, int M, int N, int K);
// Whether a residual (EPI_RESID) or store (EPI_STORE_F32) projection with
// these arguments ends in a K-slice reduce that can also write the RMSNorm of
// its rows (norm_w; a store projection then writes only the normalised rows).
bool gemm_fuses_norm(int dtype, const GemmArgs& a, int epi = EPI_RESID);
// K slices an EPI_STORE_F32 projection with these arguments leaves in a.part
// (fp32 [slices][M][N], slice z at z*M*N) when a.defer_reduce is set; 1: the
// output is in a.out as usual.
int gemm_store_slices(int dtype, const GemmArgs& a);
hipError_t launch_splitk_reduce_norm(const float* part, int ks, int M, int N, float* x,
                                     int64_t x_stride, const void* gain, void* y, int y_nck,
                                     float eps, bool residual, int y_block, hipStream_t st);
// Keys per row that the LM-head projection writes (its column blocks).
int gemm_amax_cols(int dtype, int M, int N, int K);

// A row-major source for the tiled copy: element (row, k) at
// seg[k / seg_k] + row * row_stride + k % seg_k (seg_k a multiple of the
// 16-byte fragment, row_stride in elements).
struct PackSrc {
  const void* seg[kMaxASeg];
  int nseg;
  int seg_k;
  int64_t row_stride;
};
inline PackSrc pack_src(const void* p, int K) {
  PackSrc s{};
  s.seg[0] = p;
  s.nseg = 1;
  s.seg_k = K;
  s.row_stride = K;
  return s;
}
// Tiled copy of a row-major [rows, K] matrix into dst, which holds the whole
// tiled [rows, K] matrix; padding is written as zeros.
hipError_t launch_pack_tiled(int dtype, const PackSrc& src, int rows, int K, void* dst,
                             hipStream_t st);

struct AttnArgs {
  const void* q;         // [batch][n_heads][16][head_dim] model dtype, rows >= B are zero
  const void* k;         // this layer's K cache base: [cache_batch][Hkv][cap][hd]
  const void* v;         // this layer's V cache base: [cache_batch][Hkv][cap/32][hd][32]
  const int32_t* ctx_len;
  int batch, n_heads, n_kv_heads, head_dim, block, cap;
  int window;            // > 0: query i (position ctx_len + i) sees keys p > ctx_len + i - window
  int wg_per_head;       // workgroups per KV head that split its keys (grid x)
  int min_blocks;        // fewest 32-key blocks a workgroup is given
  float scale_log2;      // log2(e) / sqrt(head_dim)
  float* part_o;         // [Hkv][wg_per_head + batch][G][hd][16]
  float* part_ml;        // [Hkv][wg_per_head + batch][G][16][2]  (running max in log2 units, sum)
  void* out;             // tiled [batch*B, n_heads*hd] model dtype (out_nck chunks per row);
  int out_nck;           // written by the partial kernel when a sequence lies in one
                         // workgroup's range, else by the combine
};

hipError_t launch_attention(int dtype, const AttnArgs& a, hipStream_t st);

// Training-pattern attention of packed blocks: block b (sequence b / nb,
// anchor position anchors[b]) attends to its sequence's context rows
// 0 .. anchor-1 in the decoding cache and to its own B keys.
struct PackedAttnArgs {
  const void* q;          // [n_blk][B][Hq][hd] model dtype
  const void* k_blk;      // [n_blk][B][Hkv][hd]
  const void* v_blk;
  const void* k;          // one layer's K cache: [cache_batch][Hkv][cap][hd]
  const void* v;          // one layer's V cache: [cache_batch][Hkv][cap/32][hd][32]
  const int32_t* ctx_len; // [cache_batch]
  const int32_t* anchors; // [n_blk]
  void* out;              // [n_blk][B][Hq][hd]
  int32_t* dev_status;
  int n_blk, blocks_per_seq, n_heads, n_kv_heads, head_dim, block, cap;
  float scale_log2;
};
hipError_t launch_packed_attention(int dtype, const PackedAttnArgs& a, hipStream_t st);

// Per-head RMSNorm + RoPE of q/k and the K/V cache scatter.
//  Forward mode (kv_rows == nullptr): src is the fused QKV output
//   [batch*B][(Hq + 2*Hkv)*hd] fp32; q heads go to q_out ([batch][Hq][16][hd],
//   rows B..15 zero-filled), k/v heads to cache position ctx_len[s] + i.
//  Append mode: src is [n_tok][n_layers * 2 * Hkv * hd] fp32 (layer-major,
//   K then V per layer); row r of sequence s goes to position
//   ctx_len[s] + r - cu_new[s] of every layer.
struct NormRopeArgs {
  const float* src;
  int64_t src_stride;
  void* q_out;
  void* k_cache;          // layer 0 base; layer stride = cache_batch*Hkv*cap*hd
  void* v_cache;
  const void* q_norm[kMaxLayers];   // per-layer gains [hd] (forward mode: only [0])
  const void* k_norm[kMaxLayers];
  const int32_t* ctx_len;
  const int32_t* cu_new;  // append mode: row offsets of each sequence's new rows
  const int32_t* accept_len;  // append mode, block rows: when non-null, row s*block + i of
                              // sequence s is appended iff i <= accept_len[s] (cu_new unused)
  int32_t* ctx_len_out;   // append mode: ctx_len (the live array, updated by the kernel);
                          // ctx_len above then points at a snapshot taken before the call
  int src_slices;         // append mode: > 1: a row of src is the sum, in slice order, of
  int64_t slice_stride;   // src_slices fp32 K-slice partials slice_stride floats apart
  int32_t* dev_status;
  int batch, cache_batch, n_heads, n_kv_heads, head_dim, block, cap, n_layers;
  int n_tok;              // append mode
  float eps;
  float rope_theta;       // <= 0: no rotation
  double inv_freq[64];    // rope_theta^(-2i / head_dim), i < head_dim / 2 (set by the launchers)
};

hipError_t launch_norm_rope_forward(int dtype, const NormRopeArgs& a, hipStream_t st);
hipError_t launch_norm_rope_append(int dtype, const NormRopeArgs& a, hipStream_t st);

// y[r] = RMSNorm(x[src_row(r)]) * gain, src_row(r) = (r / rpg) * grp_stride + grp_off + r % rpg.
// y is row-major with y_stride when y_nck == 0, else tiled [rows, d] with y_nck chunks.
hipError_t launch_rmsnorm(int dtype, const float* x, int64_t x_stride, const void* gain, void* y,
                          int64_t y_stride, int y_nck, int rows, int d, float eps, int rpg,
                          int grp_stride, int grp_off, hipStream_t st);

// Block embedding into the fp32 residual x, plus h = RMSNorm(x; gain) for
// layer 0, h tiled [batch*block, d]; zeroes arrivals[0..batch) when non-null.
hipError_t launch_embed(int dtype, const void* embed, const int32_t* anchor, int batch, int block,
                        int d, int vocab, int mask_id, float* x, const void* gain, float eps,
                        void* h, int32_t* dev_status, int32_t* arrivals, hipStream_t st);

// Draft tokens from the LM head's per-workgroup keys ([batch*(B-1)][n_cols]),
// plus the greedy accept rule when targets is non-null (arrivals: per-sequence
// counters, zero on entry, left zero).
hipError_t launch_argmax_accept(const unsigned long long* amax, int64_t stride, int n_cols,
                                int batch, int block, int32_t* drafts, const int32_t* targets,
                                int32_t* accept_len, int32_t* bonus, int32_t* arrivals,
                                hipStream_t st);

hipError_t launch_accept(const int32_t* drafts, const int32_t* targets, int batch, int block,
                         int32_t* accept_len, int32_t* bonus, int32_t* anchor_out,
                         hipStream_t st);

// ctx_len[s] += cu_new[s+1] - cu_new[s], or, when accept_len is non-null,
// ctx_len[s] += accept_len[s] + 1 (accept lengths outside [0, block) are
// clamped and flagged); clamped to cap.
hipError_t launch_ctx_len_add(int32_t* ctx_len, const int32_t* cu_new, const int32_t* accept_len,
                              int block, int batch, int n_tok, int cap, int32_t* dev_status,
                              hipStream_t st);

// Temperature > 0 drafting and verification (sampling.hip).
int sampling_splits(int vocab);
int64_t sample_ws_bytes(int rows, int vocab);
int64_t verify_ws_bytes(int batch, int block, int vocab);
hipError_t launch_sample_drafts(const float* logits, int64_t ld, int rows, int vocab, float temp,
                                uint64_t seed, int rnd, int32_t* tokens, float* logq, void* ws,
                                hipStream_t st);
hipError_t launch_verify_sampled(const int32_t* drafts, const float* draft_logits,
                                 const float* draft_logq, const float* target_logits, int batch,
                                 int block, int vocab,
                                 float temp, uint64_t seed, int rnd, int32_t* accept_len,
                                 int32_t* out_token, int32_t* anchor_out, void* ws,
                                 hipStream_t st);

// The static scratch of the allocation-free drafting call: its size, and its
// device address on the current device (looked up once per device).
int64_t sample_static_scratch_bytes();
hipError_t sample_static_scratch(void** out);

// Profiler hooks (api.hip).
void prof_begin(int kind, double bytes, double flops, hipStream_t st);
void prof_end(hipStream_t st);

}  // namespace dflash
