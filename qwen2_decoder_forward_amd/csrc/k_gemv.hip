// GEMV kernels of the decode path (M <= 8 rows, f32 activations).
//
// Every weight byte is read exactly once per call.  A wavefront owns R
// output rows; its 64 lanes cover a row with 16-byte loads (8 halves per
// lane, 1 KiB per wave instruction).  All of a wave's weight loads for a
// K batch (KB chunks of 512 halves) are issued before anything else, so the
// HBM latency overlaps the activation loads and the RMSNorm prologue; the
// binary16 values are converted to f32 in registers (weights are never
// expanded in memory).  The activation chunks a lane loads are exactly the
// ones it multiplies, and for the normed variants they also give the RMS:
// the chunks of the 64 lanes partition the row, so one wave reduction of
// their squares is the row's sum of squares.  Epilogues:
//   QKV    bias, RoPE, q write and K/V cache store (pair-packed rows)
//   RESID  h += W x                 (WO and down projections)
//   SWIGLU a = silu(gate) * up      (pair-packed gate/up rows)
//   LMHEAD logits and a per-block greedy key, folded into a per-row 64-bit
//          maximum with a relaxed device-scope atomicMax (the argmax kernel
//          that follows turns it into an index and clears it)
#include "q2_device.h"

namespace q2 {

enum { EPI_QKV = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_LMHEAD = 3 };

struct GemvP {
  const uint16_t *W;
  int N, K;  // W [N, K], K % 8 == 0
  const float *x;
  int ldx, M;
  const float *norm_w;  // RMSNorm prologue when non-null (then K is the normed width)
  float eps;
  int n_groups;  // row groups of 4 waves * R rows
  Dims d;
  QkvEpi qkv;
  float *out;
  int ldo;
  unsigned long long *best;  // LMHEAD: per-row packed maxima
  float *const *logits;      // LMHEAD: device-resident pointer to [M, V] logits (may hold null)
  float *normed_out;         // LMHEAD: f32 copy of the normed rows [M, K]
  // k_gemv1_emb: the row is the embedding of token (*emb_tok)[emb_off]
  // (row 0 and *emb_bad = 1 for an id outside [0, emb_V)), written to
  // emb_h as f32 by block 0
  const int *const *emb_tok;
  int emb_off, emb_V;
  const uint16_t *emb_E;
  float *emb_h;
  unsigned int *emb_bad;
};

template <int MT, int R, int KB, int EPI>
__global__ __launch_bounds__(256) void k_gemv(GemvP p) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int K = p.K, M = p.M, N = p.N;
  constexpr bool kResid = EPI == EPI_RESID;
  // norm gains loaded with the activations (short rows) or at their use
  constexpr bool kEarlyGain = KB <= 2;
  const bool norm = !kResid && p.norm_w != nullptr;
  const float *xsrc = p.x;
  const int ldx = p.ldx;
  float *logits = nullptr;
  if (EPI == EPI_LMHEAD) logits = *p.logits;

  float inv[MT];
  unsigned long long best[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    inv[m] = 1.0f;
    best[m] = 0ull;
  }
  // The (row, column) a lane stores in the epilogue, clamped into range so
  // that every lane's epilogue loads are issued without a branch.
  const int er = lane / MT, em = lane - er * MT;
  const int emc = em < M ? em : M - 1;

  // (do-while: the grid never exceeds the row groups, and a loop-entry test
  // would wait for its kernel-argument load before the pointers are loaded)
  int rg = blockIdx.x;
  do {
    const int row0 = (rg * 4 + wave) * R;
    // 0. The loads the epilogue needs go first: vector loads return in issue
    //    order, so waiting for them later does not wait for the weights.
    const int en = min(row0 + (er < R ? er : R - 1), N - 1);
    unsigned e_pos = 0, e_seq = 0;
    float e_ba = 0.f, e_bb = 0.f, e_old = 0.f;
    if (EPI == EPI_QKV) qkv_pair_begin(p.qkv, emc, en & ~1, e_pos, e_seq, e_ba, e_bb);
    if (kResid) e_old = p.out[(size_t)emc * p.ldo + en];

    float acc[R][MT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[r][m] = 0.f;

    QkvPair e_pair;
    for (int kb0 = 0; kb0 < K; kb0 += KB * 512) {
      const bool first = kb0 == 0;
      // 1. activations (and the norm gains, once) ahead of the weights, so the
      //    RMS reduction overlaps the weight stream; out-of-range chunks load
      //    a valid address and are zeroed
      f4 xv[KB][MT][2], gv[KB][2];
#pragma unroll
      for (int c = 0; c < KB; ++c) {
        const int k = kb0 + c * 512 + lane * 8;
        const bool kin = k < K;
        const int kc = kin ? k : K - 8;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const int mc = m < M ? m : M - 1;
          const f4 a0 = *(const f4 *)(xsrc + (size_t)mc * ldx + kc);
          const f4 a1 = *(const f4 *)(xsrc + (size_t)mc * ldx + kc + 4);
          const bool ok = kin && m < M;
          xv[c][m][0] = ok ? a0 : (f4){0.f, 0.f, 0.f, 0.f};
          xv[c][m][1] = ok ? a1 : (f4){0.f, 0.f, 0.f, 0.f};
        }
        if (kEarlyGain && norm && first) {
          const f4 g0 = *(const f4 *)(p.norm_w + kc), g1 = *(const f4 *)(p.norm_w + kc + 4);
          gv[c][0] = kin ? g0 : (f4){0.f, 0.f, 0.f, 0.f};
          gv[c][1] = kin ? g1 : (f4){0.f, 0.f, 0.f, 0.f};
        }
      }
      // 2. the weight stream: every load of this batch in flight at once
      h8 wv[KB][R];
#pragma unroll
      for (int c = 0; c < KB; ++c) {
        const int k = kb0 + c * 512 + lane * 8;
        const bool kin = k < K;
        const int kc = kin ? k : K - 8;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int n = row0 + r;
          const int nc = n < N ? n : N - 1;
          const h8 w = __builtin_nontemporal_load((const h8 *)(p.W + (size_t)nc * K + kc));
          wv[c][r] = kin && n < N ? w : (h8){0, 0, 0, 0, 0, 0, 0, 0};
        }
      }
      // 3. the epilogue's dependent loads (cos/sin at the row's position)
      if (EPI == EPI_QKV && first) e_pair = qkv_pair_end(p.d, p.qkv, emc, en & ~1, e_pos, e_seq, e_ba, e_bb);
      // 4. RMSNorm of the activations (normed variants: K <= KB * 512, one batch)
      if (norm && first) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          float ss = 0.f;
#pragma unroll
          for (int c = 0; c < KB; ++c)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              const f4 v = xv[c][m][hh];
              ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
            }
          ss = wave_sum(ss);
          inv[m] = 1.0f / sqrtf(ss / (float)K + p.eps);
        }
#pragma unroll
        for (int c = 0; c < KB; ++c) {
          if (!kEarlyGain) {  // (long rows: loaded here, keeping registers for occupancy)
            const int kc = min(c * 512 + lane * 8, K - 8);
            gv[c][0] = *(const f4 *)(p.norm_w + kc);
            gv[c][1] = *(const f4 *)(p.norm_w + kc + 4);
          }
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            xv[c][m][0] = xv[c][m][0] * inv[m] * gv[c][0];
            xv[c][m][1] = xv[c][m][1] * inv[m] * gv[c][1];
          }
        }
      }
      // 5. multiply-accumulate in f32
#pragma unroll
      for (int c = 0; c < KB; ++c)
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const float xs[8] = {xv[c][m][0].x, xv[c][m][0].y, xv[c][m][0].z, xv[c][m][0].w,
                               xv[c][m][1].x, xv[c][m][1].y, xv[c][m][1].z, xv[c][m][1].w};
#pragma unroll
          for (int r = 0; r < R; ++r)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[r][m] = fmaf((float)wv[c][r][j], xs[j], acc[r][m]);
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[r][m] = wave_sum(acc[r][m]);

    if (kResid) {
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m)
          if (lane == r * MT + m && m < M && row0 + r < N)
            p.out[(size_t)m * p.ldo + row0 + r] = e_old + acc[r][m];
    } else if (EPI == EPI_SWIGLU) {
#pragma unroll
      for (int r = 0; r < R; r += 2)
#pragma unroll
        for (int m = 0; m < MT; ++m)
          if (lane == r * MT + m && m < M && row0 + r < N)
            p.out[(size_t)m * p.ldo + ((row0 + r) >> 1)] = silu(acc[r][m]) * acc[r + 1][m];
    } else if (EPI == EPI_QKV) {
#pragma unroll
      for (int r = 0; r < R; r += 2)
#pragma unroll
        for (int m = 0; m < MT; ++m)
          if (lane == r * MT + m && m < M && row0 + r < N)
            qkv_pair_store(e_pair, acc[r][m], acc[r + 1][m]);
    } else {  // EPI_LMHEAD
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const int n = row0 + r;
          if (m < M && n < N) {
            if (logits && lane == r * MT + m) logits[(size_t)m * N + n] = acc[r][m];
            const unsigned long long key = argmax_key(acc[r][m], n);
            best[m] = key > best[m] ? key : best[m];
          }
        }
    }
    rg += gridDim.x;
  } while (rg < p.n_groups);

  if (EPI == EPI_LMHEAD) {
    __shared__ unsigned long long s_best[4][MT];
    if (lane == 0)
#pragma unroll
      for (int m = 0; m < MT; ++m) s_best[wave][m] = best[m];
    if (blockIdx.x == 0 && wave == 0 && p.normed_out) {
#pragma unroll
      for (int m = 0; m < MT; ++m)
        if (m < M)
          for (int k = lane; k < K; k += 64)
            p.normed_out[(size_t)m * K + k] = p.x[(size_t)m * p.ldx + k] * inv[m] * p.norm_w[k];
    }
    __syncthreads();
    if ((int)threadIdx.x < M && threadIdx.x < MT) {
      const int m = threadIdx.x;
      unsigned long long b = s_best[0][m];
      for (int w = 1; w < 4; ++w) b = s_best[w][m] > b ? s_best[w][m] : b;
      atomicMax(&p.best[m], b);
    }
  }
}

// One-row variant (batch-1 decode).  The block stages the activation row in
// LDS once instead of every wavefront loading all of it: thread t loads
// KB / 2 16-byte pieces of the row (and of the norm gains), issued before
// the wavefront's weight loads so their wait does not wait for the weight
// stream; the block reduces the row's sum of squares, and each thread
// writes its normed pieces.  The LDS row is laid out so that the two
// 16-byte halves of the 8-value chunk a lane multiplies sit in two
// contiguous 256-byte runs (conflict-free reads).  Weight loads, their
// f32 conversion and the epilogues are those of k_gemv.
__device__ __forceinline__ int xs_slot(int k) {  // LDS slot of element k of a batch
  const int c = k >> 9, r = k & 511;
  return (c << 9) + (((r >> 2) & 1) << 8) + ((r >> 3) << 2) + (r & 3);
}

template <int R, int KB, int EPI, bool EMB>
__device__ __forceinline__ void gemv1_body(const GemvP &p) {
  static_assert(KB % 2 == 0, "KB / 2 pieces per thread");
  static_assert(!EMB || EPI == EPI_QKV, "the embedding gather feeds the first QKV projection");
  constexpr int XP = KB / 2;  // 16-byte activation pieces per thread and batch
  __shared__ __attribute__((aligned(16))) float sx[KB * 512];
  __shared__ float sRed[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = p.K, N = p.N;
  // The kernel arguments the weight stream needs, all requested in the first
  // scalar-load batch: the empty asm uses them here, so no load of them is
  // moved into a later block (each later batch would cost a round trip before
  // the weight loads go out).
  const uint16_t *const Wp = p.W;
  const float *const xg = p.x;
  const float *const gw = p.norm_w;
  asm volatile("" ::"s"(Wp), "s"(xg), "s"(gw), "s"(K), "s"(N));
  constexpr bool kResid = EPI == EPI_RESID;
  constexpr bool norm = !kResid;  // (the QKV and gate/up launches always pass norm_w)
  const int er = lane < R ? lane : R - 1;  // the row this lane stores (lanes < R)

  // One row group per block (the launch gives every group its own block),
  // so nothing waits for a loop bound before the pointers are loaded.
  {
    const int rg = blockIdx.x;
    const int row0 = (rg * 4 + wave) * R;
    const int en = min(row0 + er, N - 1);
    unsigned e_pos = 0, e_seq = 0;
    float e_ba = 0.f, e_bb = 0.f, e_old = 0.f;
    if (EPI == EPI_QKV) qkv_pair_begin(p.qkv, 0, en & ~1, e_pos, e_seq, e_ba, e_bb);
    if (kResid) e_old = p.out[en];

    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.f;
    QkvPair e_pair;
    float inv = 1.0f;
    // (do-while: K > 0, and a loop-entry test would wait for K before the
    // pointers are loaded)
    int kb0 = 0;
    int tok = 0;  // (EMB: the token id as read)
    do {
      const bool first = kb0 == 0;
      // 1. this thread's pieces of the activation row (and gains)
      f4 xp[XP], gp[XP];
      auto load_x = [&]() {
        const _Float16 *er = nullptr;
        if constexpr (EMB) {
          tok = (*p.emb_tok)[p.emb_off];
          er = (const _Float16 *)p.emb_E + (size_t)(tok < 0 || tok >= p.emb_V ? 0 : tok) * K;
        }
#pragma unroll
        for (int i = 0; i < XP; ++i) {
          const int k = kb0 + 4 * (tid + 256 * i);
          const int kc = k < K ? k : K - 4;
          f4 a;
          if constexpr (EMB) {
            const h4 e = *(const h4 *)(er + kc);
            a = (f4){(float)e[0], (float)e[1], (float)e[2], (float)e[3]};
          } else {
            a = *(const f4 *)(xg + kc);
          }
          xp[i] = k < K ? a : (f4){0.f, 0.f, 0.f, 0.f};
          if (norm && first) {
            const f4 g = *(const f4 *)(gw + kc);
            gp[i] = k < K ? g : (f4){0.f, 0.f, 0.f, 0.f};
          }
        }
      };
      // 2. the weight stream
      h8 wv[KB][R];
      auto load_w = [&]() {
#pragma unroll
        for (int c = 0; c < KB; ++c) {
          const int k = kb0 + c * 512 + lane * 8;
          const bool kin = k < K;
          const int kc = kin ? k : K - 8;
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const int n = row0 + r;
            const int nc = n < N ? n : N - 1;
            const h8 w = __builtin_nontemporal_load((const h8 *)(Wp + (size_t)nc * K + kc));
            wv[c][r] = kin && n < N ? w : (h8){0, 0, 0, 0, 0, 0, 0, 0};
          }
        }
      };
      // (the embedded row waits for two dependent reads, the token's pointer
      // and the token: its weights are requested first)
      if constexpr (EMB) {
        load_w();
        load_x();
      } else {
        load_x();
        load_w();
      }
      if (EPI == EPI_QKV && first)
        e_pair = qkv_pair_end(p.d, p.qkv, 0, en & ~1, e_pos, e_seq, e_ba, e_bb);
      if constexpr (EMB) {
        if (blockIdx.x == 0) {  // the residual stream's row, and the id check
          // (after the epilogue's loads are requested)
#pragma unroll
          for (int i = 0; i < XP; ++i) {
            const int k = kb0 + 4 * (tid + 256 * i);
            if (k < K) *(f4 *)(p.emb_h + k) = xp[i];
          }
          if (tid == 0 && (tok < 0 || tok >= p.emb_V)) *p.emb_bad = 1u;
        }
      }
      // 3. RMS of the row over the block (normed variants: one batch)
      if (norm && first) {
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < XP; ++i) ss += xp[i].x * xp[i].x + xp[i].y * xp[i].y + xp[i].z * xp[i].z + xp[i].w * xp[i].w;
        ss = wave_sum(ss);
        if (lane == 0) sRed[wave] = ss;
        __syncthreads();
        inv = 1.0f / sqrtf(((sRed[0] + sRed[1]) + (sRed[2] + sRed[3])) / (float)K + p.eps);
#pragma unroll
        for (int i = 0; i < XP; ++i) xp[i] = xp[i] * inv * gp[i];
      } else {
        __syncthreads();  // the previous batch's LDS reads are done
      }
#pragma unroll
      for (int i = 0; i < XP; ++i) *(f4 *)(sx + xs_slot(4 * (tid + 256 * i))) = xp[i];
      __syncthreads();
      // 4. multiply-accumulate in f32
#pragma unroll
      for (int c = 0; c < KB; ++c) {
        const f4 x0 = *(const f4 *)(sx + c * 512 + lane * 4);
        const f4 x1 = *(const f4 *)(sx + c * 512 + 256 + lane * 4);
        const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[r] = fmaf((float)wv[c][r][j], xs[j], acc[r]);
      }
      kb0 += KB * 512;
    } while (kb0 < K);
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = wave_sum(acc[r]);

    if (kResid) {
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (lane == r && row0 + r < N) p.out[row0 + r] = e_old + acc[r];
    } else if (EPI == EPI_SWIGLU) {
#pragma unroll
      for (int r = 0; r < R; r += 2)
        if (lane == r && row0 + r < N) p.out[(row0 + r) >> 1] = silu(acc[r]) * acc[r + 1];
    } else if (EPI == EPI_QKV) {
#pragma unroll
      for (int r = 0; r < R; r += 2)
        if (lane == r && row0 + r < N) qkv_pair_store(e_pair, acc[r], acc[r + 1]);
    }
  }
}

template <int R, int KB, int EPI>
__global__ __launch_bounds__(256) void k_gemv1(GemvP p) {
  gemv1_body<R, KB, EPI, false>(p);
}

// The first layer's QKV projection of a one-row decode step with the
// embedding gather folded in (one launch fewer per token).
template <int R, int KB>
__global__ __launch_bounds__(256) void k_gemv1_emb(GemvP p) {
  gemv1_body<R, KB, EPI_QKV, true>(p);
}

// lm_head of the GEMV path: logits = W_lm RMSNorm(h) w_out, and each row's
// greedy key.  A persistent grid (a few blocks per CU) walks the vocabulary
// in row groups of 4 R rows per block; the normed activations are built once
// per block and kept in registers, and the weights of a block's next row
// group are requested before the current group is multiplied (two register
// sets), so the 272 MB weight stream of the 0.5B shape never drains between
// rounds.  K <= KB * 512.
template <int MT, int R, int KB>
__global__ __launch_bounds__(256) void k_lmhead(GemvP p) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int K = p.K, M = p.M, N = p.N;
  float *logits = *p.logits;

  auto wload = [&](int rg, h8 (&w)[KB][R]) {
    const int row0 = (rg * 4 + wave) * R;
#pragma unroll
    for (int c = 0; c < KB; ++c) {
      const int k = c * 512 + lane * 8;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int n = min(row0 + r, N - 1);  // (rows past N: loaded, never stored)
        if (k < K)
          w[c][r] = __builtin_nontemporal_load((const h8 *)(p.W + (size_t)n * K + k));
        else
          w[c][r] = (h8){0, 0, 0, 0, 0, 0, 0, 0};
      }
    }
  };

  int rg = blockIdx.x;
  h8 wa[KB][R];
  wload(rg, wa);

  // normed activations of the lane's chunks: x * inv_rms * w_out
  f4 xn[KB][MT][2];
  float inv[MT];
#pragma unroll
  for (int c = 0; c < KB; ++c) {
    const int k = c * 512 + lane * 8;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (k < K && m < M) {
        xn[c][m][0] = *(const f4 *)(p.x + (size_t)m * p.ldx + k);
        xn[c][m][1] = *(const f4 *)(p.x + (size_t)m * p.ldx + k + 4);
      } else {
        xn[c][m][0] = (f4){0.f, 0.f, 0.f, 0.f};
        xn[c][m][1] = (f4){0.f, 0.f, 0.f, 0.f};
      }
    }
  }
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < KB; ++c)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const f4 v = xn[c][m][hh];
        ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
      }
    inv[m] = 1.0f / sqrtf(wave_sum(ss) / (float)K + p.eps);
  }
#pragma unroll
  for (int c = 0; c < KB; ++c) {
    const int k = c * 512 + lane * 8;
    if (k < K) {
      const f4 g0 = *(const f4 *)(p.norm_w + k), g1 = *(const f4 *)(p.norm_w + k + 4);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        xn[c][m][0] = xn[c][m][0] * inv[m] * g0;
        xn[c][m][1] = xn[c][m][1] * inv[m] * g1;
      }
    }
  }

  unsigned long long best[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) best[m] = 0ull;

  for (; rg < p.n_groups; rg += gridDim.x) {
    h8 wb[KB][R];
    const bool more = rg + (int)gridDim.x < p.n_groups;  // (uniform across the block)
    if (more) wload(rg + gridDim.x, wb);
    const int row0 = (rg * 4 + wave) * R;
    float acc[R][MT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[r][m] = 0.f;
#pragma unroll
    for (int c = 0; c < KB; ++c)
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const float xs[8] = {xn[c][m][0].x, xn[c][m][0].y, xn[c][m][0].z, xn[c][m][0].w,
                             xn[c][m][1].x, xn[c][m][1].y, xn[c][m][1].z, xn[c][m][1].w};
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[r][m] = fmaf((float)wa[c][r][j], xs[j], acc[r][m]);
      }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const float v = wave_sum(acc[r][m]);
        const int n = row0 + r;
        if (m < M && n < N) {
          if (logits && lane == r * MT + m) logits[(size_t)m * N + n] = v;
          const unsigned long long key = argmax_key(v, n);
          best[m] = key > best[m] ? key : best[m];
        }
      }
    if (more) {
#pragma unroll
      for (int c = 0; c < KB; ++c)
#pragma unroll
        for (int r = 0; r < R; ++r) wa[c][r] = wb[c][r];
    }
  }

  __shared__ unsigned long long s_best[4][MT];
  if (lane == 0)
#pragma unroll
    for (int m = 0; m < MT; ++m) s_best[wave][m] = best[m];
  if (blockIdx.x == 0 && wave == 0 && p.normed_out) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
      if (m < M)
        for (int k = lane; k < K; k += 64)
          p.normed_out[(size_t)m * K + k] = p.x[(size_t)m * p.ldx + k] * inv[m] * p.norm_w[k];
  }
  __syncthreads();
  if ((int)threadIdx.x < M && threadIdx.x < MT) {
    const int m = threadIdx.x;
    unsigned long long b = s_best[0][m];
    for (int w = 1; w < 4; ++w) b = s_best[w][m] > b ? s_best[w][m] : b;
    atomicMax(&p.best[m], b);
  }
}

// ------------------------------------------------------------------ launch
template <int EPI>
constexpr bool kResidEpi() { return EPI == EPI_RESID; }

template <int R, int EPI, int MT>
static void launch_kb(GemvP &p, int grid, hipStream_t st) {
  const int kc = (p.K + 511) / 512;
  if (kc <= 2)
    hipLaunchKernelGGL((k_gemv<MT, R, 2, EPI>), dim3(grid), dim3(256), 0, st, p);
  else if (kc <= 8)
    hipLaunchKernelGGL((k_gemv<MT, R, 8, EPI>), dim3(grid), dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL((k_gemv<MT, R, 10, EPI>), dim3(grid), dim3(256), 0, st, p);
}

template <int R, int EPI>
static void launch(GemvP &p, int max_grid, hipStream_t st) {
  p.n_groups = (p.N + 4 * R - 1) / (4 * R);
  const int grid = p.n_groups < max_grid ? p.n_groups : max_grid;
  if (EPI != EPI_LMHEAD && p.M <= 1) {  // (one-row lm_head: k_lmhead)
    // k_gemv1 takes exactly one row group per block: grid = n_groups
    // (max_grid is never below n_groups on this path)
    const int kc = (p.K + 511) / 512;
    constexpr int E1 = EPI == EPI_LMHEAD ? EPI_RESID : EPI;  // (never launched for lm_head)
    // (rows longer than one batch of 10 chunks, residual only: batches of
    // 2 chunks, measured faster on the hd-128 down projection, 3584 x
    // 18944: 24.6 -> 23.0 us)
    if (kc <= 2 || (kResidEpi<E1>() && kc > 10))
      hipLaunchKernelGGL((k_gemv1<R, 2, E1>), dim3(grid), dim3(256), 0, st, p);
    else if (kc <= 4)
      hipLaunchKernelGGL((k_gemv1<R, 4, E1>), dim3(grid), dim3(256), 0, st, p);
    else if (kc <= 8)
      hipLaunchKernelGGL((k_gemv1<R, 8, E1>), dim3(grid), dim3(256), 0, st, p);
    else
      hipLaunchKernelGGL((k_gemv1<R, 10, E1>), dim3(grid), dim3(256), 0, st, p);
  } else {
    launch_kb<R, EPI, 8>(p, grid, st);
  }
}

// Matrices up to 20 MB: an eighth of one is 2.5 MB of an XCD's 4 MB L2.
constexpr long long kWarmMaxBytes = 20ll << 20;

L2Warm warm_gemv1(const uint16_t *W, int N, int K, int R, int p0, int n_prod, int max_steps) {
  L2Warm f{};
  f.base = (const uint4 *)W;
  f.total_u4 = (long long)N * K / 8;
  f.group_u4 = R * K / 2;  // 4 waves x R rows x K halves, 8 halves per 16 bytes
  f.n_groups = (N + 4 * R - 1) / (4 * R);
  f.p0 = p0;
  // the largest run of one XCD's groups a producer gets, in 256-thread steps
  const long long per_xcd = (f.n_groups + 7) / 8, prod_xcd = n_prod / 8;
  const long long steps =
      prod_xcd > 0 ? ((per_xcd + prod_xcd - 1) / prod_xcd * f.group_u4 + 255) / 256 : 0;
  const bool pays = prod_xcd > 0 && f.group_u4 >= 256 && f.total_u4 * 16 <= kWarmMaxBytes &&
                    steps <= max_steps;
  f.n_prod = pays ? n_prod : 0;
  return f;
}

static GemvP base(const uint16_t *W, int N, int K, const float *x, int ldx, int M) {
  GemvP p{};
  p.W = W;
  p.N = N;
  p.K = K;
  p.x = x;
  p.ldx = ldx;
  p.M = M;
  return p;
}

void gemv_qkv(const Dims &d, const LayerW &w, const float *h, int M, const QkvEpi &e,
              float eps, float *normed, hipStream_t st, const EmbedSrc *emb) {
  GemvP p = base(w.wqkv, d.nqkv, d.H, h, d.H, M);
  p.d = d;
  p.qkv = e;
  if (emb) {  // (callers pass it only where gemv_qkv_embeds holds)
    p.norm_w = w.attn_norm;
    p.eps = eps;
    p.emb_tok = emb->tokens;
    p.emb_off = emb->off;
    p.emb_V = emb->V;
    p.emb_E = emb->E;
    p.emb_h = const_cast<float *>(h);
    p.emb_bad = emb->bad;
    p.n_groups = (p.N + 4 * 2 - 1) / (4 * 2);
    const int kc = (p.K + 511) / 512;
    if (kc <= 2)
      hipLaunchKernelGGL((k_gemv1_emb<2, 2>), dim3(p.n_groups), dim3(256), 0, st, p);
    else if (kc <= 4)
      hipLaunchKernelGGL((k_gemv1_emb<2, 4>), dim3(p.n_groups), dim3(256), 0, st, p);
    else if (kc <= 8)
      hipLaunchKernelGGL((k_gemv1_emb<2, 8>), dim3(p.n_groups), dim3(256), 0, st, p);
    else
      hipLaunchKernelGGL((k_gemv1_emb<2, 10>), dim3(p.n_groups), dim3(256), 0, st, p);
    return;
  }
  if (d.H > kGemvNormCols) {  // wide rows: norm first, then the multi-batch GEMV
    rmsnorm_rows_f16(const_cast<float *>(h), d.H, w.attn_norm, d.H, M, eps, nullptr, 0, normed,
                     nullptr, 0, st);
    p.x = normed;
    p.n_groups = (p.N + 4 * 2 - 1) / (4 * 2);
    hipLaunchKernelGGL((k_gemv<8, 2, 10, EPI_QKV>), dim3(p.n_groups), dim3(256), 0, st, p);
    return;
  }
  p.norm_w = w.attn_norm;
  p.eps = eps;
  launch<2, EPI_QKV>(p, 1 << 30, st);
}

void gemv_resid(const uint16_t *W, int N, int K, const float *x, int ldx, int M, float *h,
                int ldh, hipStream_t st) {
  GemvP p = base(W, N, K, x, ldx, M);
  p.out = h;
  p.ldo = ldh;
  if (down_rows1(K) == 1)
    launch<1, EPI_RESID>(p, 1 << 30, st);
  else
    launch<2, EPI_RESID>(p, 1 << 30, st);
}

void gemv_swiglu(const Dims &d, const LayerW &w, const float *h, int M, float *a, int lda,
                 float eps, float *normed, hipStream_t st) {
  GemvP p = base(w.wgu, 2 * d.I_pad, d.H, h, d.H, M);
  p.out = a;
  p.ldo = lda;
  if (d.H > kGemvNormCols) {  // wide rows: norm first, then the multi-batch GEMV
    rmsnorm_rows_f16(const_cast<float *>(h), d.H, w.ffn_norm, d.H, M, eps, nullptr, 0, normed,
                     nullptr, 0, st);
    p.x = normed;
    p.n_groups = (p.N + 4 * 4 - 1) / (4 * 4);
    hipLaunchKernelGGL((k_gemv<8, 4, 10, EPI_SWIGLU>), dim3(p.n_groups), dim3(256), 0, st, p);
    return;
  }
  p.norm_w = w.ffn_norm;
  p.eps = eps;
  // (one row: pairs of rows per wave, twice the blocks of 4-row waves; the
  // 0.5B gate/up GEMV measured 5.94 -> 5.36 us)
  if (M <= 1)
    launch<kGateUpRows1, EPI_SWIGLU>(p, 1 << 30, st);
  else
    launch<4, EPI_SWIGLU>(p, 1 << 30, st);
}

template <int MT, int R, int KB>
static void launch_lmhead(GemvP &p, hipStream_t st) {
  p.n_groups = (p.N + 4 * R - 1) / (4 * R);
  const int grid = p.n_groups < 1024 ? p.n_groups : 1024;  // 4 blocks per CU
  hipLaunchKernelGGL((k_lmhead<MT, R, KB>), dim3(grid), dim3(256), 0, st, p);
}

void gemv_lmhead(const Dims &d, const uint16_t *W, const float *norm_w, const float *h, int M,
                 float *normed_out, const ArgmaxEpi &e, float eps, hipStream_t st) {
  GemvP p = base(W, d.V, d.H, h, d.H, M);
  p.norm_w = norm_w;
  p.eps = eps;
  p.best = e.best;
  p.logits = e.logits;
  p.normed_out = normed_out;
  const int kc = (d.H + 511) / 512;  // 512-half chunks per row
  if (d.H > kGemvNormCols) {  // wide rows: the final norm first (it also gives the tap)
    rmsnorm_rows_f16(const_cast<float *>(h), d.H, norm_w, d.H, M, eps, nullptr, 0, normed_out,
                     nullptr, 0, st);
    p.x = normed_out;
    p.norm_w = nullptr;
    p.normed_out = nullptr;
    launch<4, EPI_LMHEAD>(p, 4096, st);
  } else if (M <= 1) {  // one row: the persistent kernel (its normed row stays in registers)
    if (kc <= 2) launch_lmhead<1, 4, 2>(p, st);
    else if (kc <= 4) launch_lmhead<1, 2, 4>(p, st);
    else if (kc <= 8) launch_lmhead<1, 1, 8>(p, st);
    else launch_lmhead<1, 1, 10>(p, st);
  } else {  // up to 8 rows: the GEMV kernel (8 normed rows would not fit in registers)
    launch<4, EPI_LMHEAD>(p, 4096, st);
  }
  argmax_finalize(e, M, st);
}

}  // namespace q2
