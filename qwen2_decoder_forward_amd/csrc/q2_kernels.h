// Internal interface between the host runtime (qwen2_abi.cpp) and the HIP
// kernels (k_*.hip).  Not part of the public C ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <string>

namespace q2 {

// Model dimensions as the kernels see them.
struct Dims {
  int L, H, nh, nkv, hd, group, I, I_pad, V, n_ctx, n_seq;
  int nqkv;  // (nh + 2 * nkv) * hd rows of the fused QKV matrix
};

// Device weight store of one layer (repacked at load time).
//  wqkv [nqkv, H]: rows [q heads | k heads | v heads]; inside every head the
//       rows are pair-interleaved: packed rows (2j, 2j+1) hold the natural
//       rows (j, j + hd/2), the two halves RoPE rotates together.
//  bqkv [nqkv] in the same packed order.
//  wgu  [2 * I_pad, H]: packed row 2i = gate row i, 2i+1 = up row i; rows of
//       i >= I are zero.
//  wd   [H, I_pad]: columns >= I are zero.
struct LayerW {
  const float *attn_norm, *ffn_norm, *bqkv;
  const uint16_t *wqkv, *wo, *wgu, *wd;
};

// Where rows of the current call live and where K/V go.
struct RowInfo {
  const int *pos;  // [M] position of each row
  const int *seq;  // [M] sequence slot of each row
};

// The f32 cache is the one decode attention reads; every K/V store also
// writes a binary16 mirror laid out for the MFMA prefill attention: K as
// [L][n_seq][nkv][ldp][hd] and V transposed as [L][n_seq][nkv][hd][ldp],
// ldp = n_ctx rounded up to 64 positions (zero where nothing was written).
struct KVCache {
  float *k, *v;  // [L][n_seq][nkv][n_ctx][hd] each
  _Float16 *k16, *v16t;
  int ldp;
  __host__ __device__ size_t off(const Dims &d, int l, int s, int g, int p) const {
    return ((((size_t)l * d.n_seq + s) * d.nkv + g) * d.n_ctx + p) * (size_t)d.hd;
  }
  // start of the (l, s, g) block of either mirror
  __host__ __device__ size_t off16(const Dims &d, int l, int s, int g) const {
    return (((size_t)l * d.n_seq + s) * d.nkv + g) * (size_t)ldp * d.hd;
  }
};

struct RopeTable {
  const float *cos, *sin;  // [n_ctx][hd/2]
};

// Epilogue of the fused QKV projection: bias, RoPE on q/k, K/V store.
struct QkvEpi {
  const float *bias;  // packed order
  float *q;           // [M, nh*hd] rotated queries (f32)
  int ldq;
  KVCache kv;
  int layer;
  RowInfo rows;
  RopeTable rope;
};

// Warming of a later launch's weights in the L2 of the XCD that will read
// them.  Blocks of a launch are dealt to the 8 XCDs round-robin by linear
// block id (block b runs on XCD b % 8), and each XCD has its own L2, so a
// one-row GEMV whose block g reads row group g reads it on XCD g % 8.  The
// one-row attention launch, whose head blocks leave HBM mostly idle (their
// K / V come from L2), takes extra producer blocks that read, on each XCD,
// the groups the same layer's down GEMV will read there; that GEMV then
// finds them in its L2.  Performance only: the producers write nothing, and
// a group they miss is read from HBM.
struct L2Warm {
  const uint4 *base;   // the later GEMV's matrix: group g starts at base + g * group_u4
  long long total_u4;  // its size in 16-byte units
  int group_u4;        // 16-byte units per group (>= 256)
  int n_groups;        // groups (the later launch's block g reads group g)
  int p0, n_prod;      // producer block ids [p0, p0 + n_prod) of the warming launch
};
// Producer blocks of the one-row attention, which warms the same layer's
// down projection, and their step bound (16-byte loads per thread).  More
// producers than idle CUs keep each one's share small: a CU pulls only about
// 26 KB per microsecond from HBM (outstanding misses over the latency).
constexpr int kWarmProdAttn = 256, kWarmStepsAttn = 16;
constexpr int kWarmProdQkv = 64;  // producers for the next layer's QKV rows
// n_prod producers for a later one-row GEMV over W [N, K] with R rows per
// wave, hosted by a launch whose producer block ids start at p0; none (n_prod
// = 0 in the result) when it does not pay (weights too large for the L2s)
// or a producer's share would exceed max_steps steps.
L2Warm warm_gemv1(const uint16_t *W, int N, int K, int R, int p0, int n_prod, int max_steps);
// Rows per wave of the one-row gate/up and down GEMVs.
constexpr int kGateUpRows1 = 2;
constexpr int down_rows1(int K) { return K >= 2048 ? 1 : 2; }

// Debug checks of a call (contexts loaded with QWEN2_DEBUG_CHECKS=1).
// mask [n_seq][n_ctx]: 1 for the slots the call may write.  debug_kv adds a
// hash of every cache word outside those slots (f32 K and V, both binary16
// mirrors) into *hash and keeps, in *bad_k / *bad_v, the smallest f32 word
// index of a non-finite K / V value inside them; debug_nonfinite keeps the
// smallest index of a non-finite value of x[0 .. n) in *bad.
struct DebugKv {
  const unsigned char *mask;
  int hd, n_ctx, ldp, nkv, n_seq;
};
void debug_kv(const DebugKv &a, const float *k, const float *v, const _Float16 *k16,
              const _Float16 *v16t, size_t f32_words, size_t f16_words,
              unsigned long long *hash, unsigned long long *bad_k, unsigned long long *bad_v,
              hipStream_t st);
void debug_nonfinite(const float *x, size_t n, unsigned long long *bad, hipStream_t st);

// Greedy readout: packed (ordered-key, ~index) 64-bit maxima per row, zero
// between calls (the finalize kernel clears them).  The output pointers are
// read on the device from a slot the host staged with the call, so a
// captured graph can write to a different buffer on every replay.
struct ArgmaxEpi {
  float *const *logits;      // -> [M, V] f32 or null
  unsigned long long *best;  // [M]
  int *const *out;           // -> [M] int32 or null
  RowInfo rows;              // position and sequence slot of each read-out row
  const int *stop;           // [1 + kMaxStopIds]: count, then the stop ids
  unsigned *stop_pos;        // [n_seq]: smallest read-out position whose id was a stop id (~0u: none)
};
constexpr int kMaxStopIds = 8;

// ---------------------------------------------------------------- launchers
// GEMV family (rows M <= 8, f32 activations, f16 weights streamed once).
// y[m, n] = sum_k x'[m, k] W[n, k] with x' = x, or RMSNorm(x) * norm_w when
// norm_w is given (then K must equal the normed width).  Rows wider than
// kGemvNormCols are normed first by k_rmsnorm_rows into `normed` ([M, H]
// f32 scratch), then multiplied by the GEMV without its norm prologue.
constexpr int kGemvNormCols = 10 * 512;
// The embedding gather folded into the first QKV projection (one row,
// rows up to kGemvNormCols): h = f32(E[(*tokens)[off]]), written by the
// same launch; an id outside [0, V) reads row 0 and sets *bad.
struct EmbedSrc {
  const uint16_t *E;
  int V;
  const int *const *tokens;
  int off;
  unsigned int *bad;
};
inline bool gemv_qkv_embeds(const Dims &d, int M) { return M == 1 && d.H <= kGemvNormCols; }
void gemv_qkv(const Dims &d, const LayerW &w, const float *h, int M, const QkvEpi &e,
              float eps, float *normed, hipStream_t st, const EmbedSrc *emb = nullptr);
void gemv_resid(const uint16_t *W, int N, int K, const float *x, int ldx, int M, float *h,
                int ldh, hipStream_t st);
void gemv_swiglu(const Dims &d, const LayerW &w, const float *h, int M, float *a, int lda,
                 float eps, float *normed, hipStream_t st);
void gemv_lmhead(const Dims &d, const uint16_t *W, const float *norm_w, const float *h, int M,
                 float *normed_out, const ArgmaxEpi &e, float eps, hipStream_t st);

// Writes the index of each row's packed maximum and clears it, and latches
// stop ids; launched after an lm_head kernel.
void argmax_finalize(const ArgmaxEpi &e, int M, hipStream_t st);
// Between natural K rows [rows, hd] and the rotation-pair order an
// Interleaved-RoPE model keeps in its cache (2j -> j, 2j+1 -> j + hd/2).
void pair_order(const float *src, float *dst, int rows, int hd, bool to_pairs, hipStream_t st);
// out[s] = the latched stop position of slot s, -1 for none (reset with clear).
void read_stops(unsigned *stop_pos, int n, int *out, int clear, hipStream_t st);
// probs[r] = softmax(logits[r]) for rows r < rows, over V columns; part holds
// rows * kProbBlocks (max, sum) pairs.
constexpr int kProbBlocks = 256;
int softmax_blocks(int rows);  // blocks per row softmax_rows uses
void softmax_rows(const float *logits, int rows, int V, float2 *part, float *probs,
                  hipStream_t st);
// Message for qwen2_last_error(NULL) from a call that has no context.
void set_static_error(const std::string &msg);

// MFMA GEMM family (rows M > 8): A f16 [M, lda], W f16 [N, K], K % 32 == 0.
// Residual GEMMs with few output tiles split K over blocks: with fewer than
// 512 rows the blocks add their f32 partial sums into h with float atomics;
// with more, the partial sums go to a context-owned workspace and the next
// RMSNorm folds them in.
struct Workspace {
  float *buf;
  size_t bytes;
};
constexpr int kMaxSplits = 16;  // split-K partial-sum sets a residual GEMM may leave
void gemm_qkv(const Dims &d, const LayerW &w, const _Float16 *x, int lda, int M,
              const QkvEpi &e, const Workspace &ws, hipStream_t st);
// The same with the attention RMSNorm fused in: the rows of h [M, ldh] are
// normed inside the GEMM (no x buffer).  Only where qkv_fuses_norm holds:
// the projection runs on the skinny kernel with 32-row tiles (fewer than 512
// rows, K <= 1024, N <= 2048).  The caller must have no split-K partial sums
// pending in h.
bool qkv_fuses_norm(const Dims &d, int M, const Workspace &ws);
void gemm_qkv_normed(const Dims &d, const LayerW &w, const float *h, int ldh, int M, float eps,
                     const QkvEpi &e, hipStream_t st);
// Returns the number of split-K partial-sum sets left in ws.buf ([z][M][N]);
// when nonzero the next rmsnorm_rows_f16 of h must fold them in.
int gemm_resid(const uint16_t *W, int N, int K, const _Float16 *x, int lda, int M, float *h,
               int ldh, const Workspace &ws, hipStream_t st);
void gemm_swiglu(const Dims &d, const LayerW &w, const _Float16 *x, int lda, int M,
                 _Float16 *a, int ld_a, const Workspace &ws, hipStream_t st);
void gemm_lmhead(const Dims &d, const uint16_t *W, const _Float16 *x, int lda, int M,
                 const ArgmaxEpi &e, hipStream_t st);

// RMSNorm of rows into an f16 copy (the MFMA A operand) and, when y32 is
// given, also into f32 [M, H].  `splits` pending partial-sum sets part[z][M][H]
// of a residual GEMM are added into h first (H <= 8192); x may be null.
void rmsnorm_rows_f16(float *h, int ldh, const float *w, int H, int M, float eps, _Float16 *x,
                      int ldx, float *y32, const float *part, int splits, hipStream_t st);
// Embedding gather h[m] = f32(E[tokens[m]]) without scaling; an id outside
// [0, V) reads row 0 and sets *bad_flag to 1.
void embed_rows(const uint16_t *E, int H, int V, const int *const *tokens, int tok_off, int M,
                float *h, unsigned int *bad_flag, hipStream_t st);
// dst[dst_rows[i]] = src[src_rows[i]] (ncols floats) for the k listed pairs;
// the row lists live on the device.
void copy_rows(const float *src, int lds, const int *src_rows, float *dst, int ldd,
               const int *dst_rows, int k, int ncols, hipStream_t st);

// Attention.
constexpr int kChunkKeys = 64;  // keys per block of the decode attention
constexpr int kMaxMergeChunks = 2048;  // chunks the merge kernel holds: n_ctx <= 131072
// A chunk record holds, for the group's query heads, the un-normalised
// outputs o[group][hd], then the maxima m[group] and exp-sums l[group],
// padded to a multiple of 4 floats (16-byte aligned records).
__host__ __device__ constexpr int attn_rec_floats(int group, int hd) {
  return (group * (hd + 2) + 3) / 4 * 4;
}
struct AttnPartials {
  float *buf;    // [rows][nkv][n_chunks] records of attn_rec_floats(group, hd)
  int n_chunks;  // chunk slots per row: ceil(n_ctx / kChunkKeys)
};
// Split-KV attention, one row per query token (decode and short prefills).
// n_chunks = ceil((max position of the rows + 1) / kChunkKeys).  With one
// chunk the output is written directly; otherwise the chunk records are
// merged by the merge kernel when `merge` (else left in the records).
void attn_decode(const Dims &d, int layer, const KVCache &kv, const float *q, int ldq,
                 RowInfo rows, int M, int n_chunks, bool merge, const AttnPartials &p,
                 float *o32, _Float16 *o16, int ldo, hipStream_t st);
// Attention fused with WO + residual for M <= 8 rows at positions below
// kFusedKeys: per (WO row chunk, query head) block, partial row sums added
// into h with float atomics.  A block's WO chunk is 4 wavefronts x
// wo_loads_per_wave(hd) loads x 512 / hd rows: hd 64 takes 64-row chunks, so
// 14 heads x 14 chunks of the 0.5B shape spread the (repeated) K/V reads of
// a head over 196 blocks (measured faster than 32, 128 or 256 rows).  Every
// block reads all of its head's keys, so from about 512 positions on the
// chunked attention with merge_wo is faster (0.5B decode at positions
// 400 / 700: 1,857 / 1,631 tok/s fused against 1,782 / 1,729 chunked).
// One-row calls (M = 1) give the row's sequence slot seq1 and a key bound
// nk1 (position < nk1 <= n_ctx) from the host: the kernel then addresses
// K / V without waiting for the row data it reads on the device.
constexpr int kFusedKeys = 512;
constexpr int wo_loads_per_wave(int hd) { return hd == 64 ? 2 : 8; }
constexpr int wo_loads_fused(int hd) { return hd == 64 ? 2 : 8; }  // (attn_wo_fused's blocks)
// warm_wd: the down projection of the same layer, warm_wqkv: the QKV
// projection of the next layer, warmed by producer blocks of the one-row
// kernel (null: none).
void attn_wo_fused(const Dims &d, int layer, const KVCache &kv, const float *q, int ldq,
                   RowInfo rows, int M, int seq1, int nk1, const uint16_t *wo, float *h, int ldh,
                   const uint16_t *warm_wd, const uint16_t *warm_wqkv, hipStream_t st);
// The chunk records of attn_decode (merge = false) of M <= 8 rows merged
// and multiplied by WO, the partial row sums added into h with float
// atomics: per (WO row chunk, query head) block as in attn_wo_fused.
void merge_wo(const Dims &d, const AttnPartials &p, RowInfo rows, int M, const uint16_t *wo,
              float *h, int ldh, hipStream_t st);
// Causal flash attention over MFMA for one prefill pass, on the binary16
// mirror of the cache.  The pass's rows are runs of one sequence each
// (segs: rows r0 .. r0+n-1 of sequence seq, positions strictly increasing
// within a run); host_pos is the host copy of the pass's positions, which
// sizes the work split.  Up to 8 runs share a launch.  Long passes use `ws`
// for the split query tiles' partial softmax states.
struct PrefillSeg {
  int r0, n, seq;
};
void attn_prefill(const Dims &d, int layer, const KVCache &kv, const float *q, int ldq,
                  RowInfo rows, const PrefillSeg *segs, int n_segs, const int *host_pos,
                  const Workspace &ws, _Float16 *o16, int ldo, hipStream_t st);
// Rewrites the binary16 mirror of positions pos0 .. pos0+n-1 of (layer, seq)
// from the f32 cache (after a direct write of the f32 cache).
void kv_mirror(const Dims &d, const KVCache &kv, int layer, int seq, int pos0, int n,
               hipStream_t st);

}  // namespace q2
