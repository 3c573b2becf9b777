// MFMA GEMMs of the prefill and batched-decode projections (rows M > 8):
//   C[M, N] = A[M, K] * W[N, K]^T,  A and W binary16, f32 accumulation,
// on v_mfma_f32_32x32x16_f16, with the projection's op fused into the
// epilogue:
//   QKV    bias + RoPE + q write / K,V cache store (pair partner via lane^1)
//   RESID  h += C                (WO, down)
//   SWIGLU a = silu(gate) * up   (pair-packed gate/up rows, f16 out)
//   LMHEAD logits + per-row greedy argmax key
// k_gemm_big (QKV, RESID, SWIGLU) uses 64-wide K slices double-buffered in
// LDS, staged through registers; k_gemm_xl (the long-K residual and SwiGLU
// GEMMs of many rows) loads 256 x 256 x 64 tiles straight into LDS;
// k_gemm_lmhead (the lm_head over the vocabulary, M <= a few hundred rows)
// uses 128 x 128 x 32 tiles staged through registers.
// MFMA 32x32 layout: lane l supplies A[l%32][8*(l/32)..+8] and
// B[8*(l/32)..+8][l%32]; it receives D[8*(r/4) + 4*(l/32) + r%4][l%32].
#include "q2_device.h"

namespace q2 {

enum { G_QKV = 0, G_RESID = 1, G_SWIGLU = 2, G_LMHEAD = 3 };

// k_gemm_lmhead: block tile LBM x 128 x 32 (LBM = 64 or 128 rows), four
// wavefronts in a 2 x 2 arrangement, each owning (LBM / 2) x 64 (LBM / 64 x
// 2 MFMA tiles); a ring of kStages register sets keeps the global loads of
// the next slices in flight while one slice is multiplied out of LDS.
constexpr int BN = 128, BK = 32, LDT = BK + 8;
constexpr int kStages = 4;  // K slices in flight per block

struct GemmP {
  const _Float16 *A;
  int lda, M;
  const _Float16 *W;
  int N, K;
  Dims d;
  QkvEpi qkv;
  float *h;
  int ldh;
  _Float16 *a16;
  int ld_a;
  ArgmaxEpi am;
  float *ws;      // split-K: raw partial sums [splits][M][N] (RESID only)
  int k_steps;    // K slices per block (per split)
  int atomic_out; // split-K residual: partial sums added into h with float atomics
  // RMSNorm fused into the skinny QKV GEMM: A = RMSNorm(hx rows) * gain,
  // built from the f32 residual rows hx [M, ldhx] (then A is unused)
  const float *hx, *gain;
  int ldhx;
  float eps;
};

template <int LBM>
__global__ __launch_bounds__(256) void k_gemm_lmhead(GemmP p) {
  constexpr int TMW = LBM / 64;  // MFMA tiles per wavefront along M
  constexpr int WTM = LBM / 2;   // wavefront tile rows
  __shared__ __attribute__((aligned(16))) _Float16 sA[LBM * LDT];
  __shared__ __attribute__((aligned(16))) _Float16 sW[BN * LDT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * LBM, n0 = blockIdx.x * BN;
  const int M = p.M, N = p.N, K = p.K;
  const int hi = lane >> 5, l32 = lane & 31;

  // each thread moves LBM / 64 16-byte chunks of A and two of W per K slice;
  // rows past M or N are clamped to the last row (their results are never
  // stored), so every load is unconditional
  const int cr0 = tid >> 2, cr1 = (tid + 256) >> 2, ck = (tid & 3) * 8;
  const _Float16 *Ap0 = p.A + (size_t)min(m0 + cr0, M - 1) * p.lda + ck;
  const _Float16 *Ap1 = p.A + (size_t)min(m0 + (LBM == 128 ? cr1 : cr0), M - 1) * p.lda + ck;
  const _Float16 *Wp0 = p.W + (size_t)min(n0 + cr0, N - 1) * K + ck;
  const _Float16 *Wp1 = p.W + (size_t)min(n0 + cr1, N - 1) * K + ck;

  f16x acc[TMW][2];
#pragma unroll
  for (int i = 0; i < TMW; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // K slices kt0 .. kt0 + nk - 1; a ring of kStages register sets keeps the
  // global loads of the next kStages - 1 slices in flight while one slice is
  // multiplied out of LDS.  Every stage issues the same loads (past the last
  // slice they re-read it) in a fixed order, so the count of outstanding
  // loads at the loop head stays exact instead of draining the ring.
  const int kt0 = blockIdx.z * p.k_steps;
  const int nk = min(K / BK - kt0, p.k_steps);
  h8 ra[kStages][2], rw[kStages][2];
  auto gl = [&](int st, int kt) {
    const int ko = (kt0 + min(kt, nk - 1)) * BK;
    ra[st][0] = *(const h8 *)(Ap0 + ko);
    if (LBM == 128) ra[st][1] = *(const h8 *)(Ap1 + ko);
    rw[st][0] = *(const h8 *)(Wp0 + ko);
    rw[st][1] = *(const h8 *)(Wp1 + ko);
  };
#pragma unroll
  for (int st = 0; st < kStages; ++st) {
    gl(st, st);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int kb = 0; kb < nk; kb += kStages) {
#pragma unroll
    for (int st = 0; st < kStages; ++st) {
      const int kt = kb + st;
      // (stages past the last slice still write, wait and load, and only
      // skip the multiply, so the loop has no branch around a load)
      *(h8 *)(sA + cr0 * LDT + ck) = ra[st][0];
      if (LBM == 128) *(h8 *)(sA + cr1 * LDT + ck) = ra[st][1];
      *(h8 *)(sW + cr0 * LDT + ck) = rw[st][0];
      *(h8 *)(sW + cr1 * LDT + ck) = rw[st][1];
      __syncthreads();
      gl(st, kt + kStages);
      __builtin_amdgcn_sched_barrier(0);
      if (kt < nk) {  // uniform across the block
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          h8 af[TMW], bf[2];
#pragma unroll
          for (int i = 0; i < TMW; ++i)
            af[i] = *(const h8 *)(sA + (wm * WTM + i * 32 + l32) * LDT + s * 16 + hi * 8);
#pragma unroll
          for (int j = 0; j < 2; ++j)
            bf[j] = *(const h8 *)(sW + (wn * 64 + j * 32 + l32) * LDT + s * 16 + hi * 8);
#pragma unroll
          for (int i = 0; i < TMW; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
      }
      __syncthreads();
    }
  }

  // ------------------------------------------ epilogue: logits + argmax key
  __shared__ unsigned long long sBest[2][LBM];
  float *logits = *p.am.logits;
  unsigned long long kb[TMW][16];
#pragma unroll
  for (int i = 0; i < TMW; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + wm * WTM + i * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
      unsigned long long b = 0ull;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = n0 + wn * 64 + j * 32 + l32;
        if (m < M && n < N) {
          const float v = acc[i][j][r];
          if (logits) logits[(size_t)m * N + n] = v;
          const unsigned long long key = argmax_key(v, n);
          b = key > b ? key : b;
        }
      }
#pragma unroll
      for (int o = 1; o < 32; o <<= 1) {
        const unsigned long long x = shfl_xor_u64(b, o);
        b = x > b ? x : b;
      }
      kb[i][r] = b;
    }
  if (l32 == 0) {
#pragma unroll
    for (int i = 0; i < TMW; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) sBest[wn][wm * WTM + i * 32 + 8 * (r >> 2) + 4 * hi + (r & 3)] = kb[i][r];
  }
  __syncthreads();
  if (tid < LBM && m0 + tid < M) {
    const unsigned long long b = sBest[0][tid] > sBest[1][tid] ? sBest[0][tid] : sBest[1][tid];
    atomicMax(&p.am.best[m0 + tid], b);
  }
}

// Epilogue of one 32 x 32 MFMA tile held by a wavefront (lane l holds
// D[8 (r/4) + 4 (l/32) + r%4][l%32], r = 0..15) whose first row is mt0 and
// whose column is n.  Every load (the residual rows, the QKV epilogue's
// tables) is issued before the first store, so the tile costs one or two
// memory round trips: a load after a store to a possibly aliasing address
// would wait for it.  Split-K residual blocks (p.ws) either add their
// partial sums into h with float atomics (p.atomic_out: GEMMs of fewer than
// 512 rows, where the adds are few; their order varies from run to run by
// an ulp) or store them raw, [split][M][N], for the next RMSNorm to fold in
// (the large-M GEMMs, whose millions of adds cost more than the fold:
// hd-128 2048-row prefill 32.7 -> 34.5 ms with atomics).
template <int EPI>
__device__ __forceinline__ void tile_epilogue(const GemmP &p, const f16x &v, int mt0, int n) {
  const int lane = threadIdx.x & 63, hi = lane >> 5;
  const int M = p.M, N = p.N;
  int m[16];
  bool ok[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    m[r] = mt0 + 8 * (r >> 2) + 4 * hi + (r & 3);
    ok[r] = m[r] < M && n < N;
    m[r] = min(m[r], M - 1);
  }
  // (residual and workspace addresses as 32-bit byte offsets from the
  // block-uniform base: h holds at most 8192 rows of 8192 floats, the
  // workspace 64 MB, so the base stays in scalar registers and a row costs
  // one vector register instead of a 64-bit pointer)
  char *const hb = (char *)p.h;
  if (EPI == G_RESID && p.ws && p.atomic_out) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (ok[r]) atomicAdd((float *)(hb + ((unsigned)m[r] * (unsigned)p.ldh + (unsigned)n) * 4u), v[r]);
  } else if (EPI == G_RESID && p.ws) {
    char *const wb = (char *)p.ws;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (ok[r])
        *(float *)(wb + (((unsigned)blockIdx.z * (unsigned)M + (unsigned)m[r]) * (unsigned)N + (unsigned)n) * 4u) = v[r];
  } else if (EPI == G_RESID) {
    const int nc = min(n, N - 1);
    float old[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) old[r] = *(const float *)(hb + ((unsigned)m[r] * (unsigned)p.ldh + (unsigned)nc) * 4u);
    pin_regs(old);
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (ok[r]) *(float *)(hb + ((unsigned)m[r] * (unsigned)p.ldh + (unsigned)n) * 4u) = old[r] + v[r];
  } else {
    float a[16], b[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      a[r] = v[r];
      b[r] = __shfl_xor(v[r], 1, 64);  // the pair partner (column n + 1)
      ok[r] = ok[r] && (n & 1) == 0;
    }
    if (EPI == G_QKV) {
      qkv_store_rows<16>(p.d, p.qkv, m, min(n & ~1, N - 2), a, b, ok);
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (ok[r]) p.a16[(size_t)m[r] * p.ld_a + (n >> 1)] = (_Float16)(silu(a[r]) * b[r]);
    }
  }
}

// f32 block tile in LDS for the QKV epilogue: element (r, c) of a BNT-wide
// row, with 16-byte chunk c/4 stored at chunk (c/4) ^ (r % (BNT/4)) so the
// column-wise writes from the MFMA layout spread over the banks.
template <int BNT>
__device__ __forceinline__ int qkv_tile_idx(int r, int c) {
  return r * BNT + ((((c >> 2) ^ r) & (BNT / 4 - 1)) << 2) + (c & 3);
}

// QKV epilogue from the block tile T (rows m0.., packed columns n0..; the
// tile is head-aligned: BNT is a multiple of head_dim).
// Pass 1: item = (row, 4 consecutive pairs) -> bias, RoPE on q / k, then
//   the natural dims d..d+3 and d+half..d+half+3 of the q row or the K / V
//   cache slot go out as two 16-byte stores (K also two 8-byte binary16
//   stores into its mirror).
// Pass 2: the transposed binary16 V mirror [d][position], with consecutive
//   lanes on consecutive rows (positions), so its 2-byte stores coalesce.
// Each pass issues all of a thread's position / table loads before its
// stores (a load behind a store to a possibly aliasing address waits for
// it).
template <int BMT, int BNT, int NT>
__device__ __forceinline__ void qkv_epilogue_lds(const GemmP &p, const float *T, int m0, int n0) {
  const Dims &d = p.d;
  const QkvEpi &e = p.qkv;
  const int tid = threadIdx.x;
  const int M = p.M, N = p.N, hd = d.hd, half = hd >> 1;
  constexpr int IPR = BNT / 8;  // items per row
  constexpr int PER = BMT * IPR / NT;
  static_assert(BMT * IPR % NT == 0, "items per thread");
  // pass 1
  int mi[PER];
  unsigned ps[PER], sq[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int item = tid + NT * k;
    mi[k] = min(m0 + item / IPR, M - 1);
    ps[k] = (unsigned)e.rows.pos[mi[k]];
    sq[k] = (unsigned)e.rows.seq[mi[k]];
  }
  f4 cs[PER], sn[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int item = tid + NT * k;
    const int n = min(n0 + 8 * (item % IPR), N - 8);
    const int head = n / hd;
    const int jd = (n - head * hd) >> 1;
    const size_t t = (size_t)ps[k] * half + jd;
    cs[k] = *(const f4 *)(e.rope.cos + t);
    sn[k] = *(const f4 *)(e.rope.sin + t);
  }
  pin_regs(sq);
  pin_regs(cs);
  pin_regs(sn);
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int item = tid + NT * k;
    const int r = item / IPR, c0 = 8 * (item % IPR);
    const int n = n0 + c0;
    if (m0 + r >= M || n >= N) continue;
    const int head = n / hd;
    const int jd = (n - head * hd) >> 1;
    const bool is_q = head < d.nh, is_k = !is_q && head < d.nh + d.nkv;
    const f4 t0 = *(const f4 *)(T + qkv_tile_idx<BNT>(r, c0));
    const f4 t1 = *(const f4 *)(T + qkv_tile_idx<BNT>(r, c0 + 4));
    const f4 b0 = *(const f4 *)(e.bias + n), b1 = *(const f4 *)(e.bias + n + 4);
    const f4 a = {t0.x + b0.x, t0.z + b0.z, t1.x + b1.x, t1.z + b1.z};  // dims jd..jd+3
    const f4 b = {t0.y + b0.y, t0.w + b0.w, t1.y + b1.y, t1.w + b1.w};  // dims jd+half..
    f4 x = a, y = b;
    if (!(head >= d.nh + d.nkv)) {
      x = a * cs[k] - b * sn[k];
      y = b * cs[k] + a * sn[k];
    }
    if (is_q) {
      float *dst = e.q + (size_t)mi[k] * e.ldq + (size_t)head * hd + jd;
      *(f4 *)dst = x;
      *(f4 *)(dst + half) = y;
    } else {
      const size_t g = (size_t)(is_k ? head - d.nh : head - d.nh - d.nkv);
      const size_t blk = ((size_t)e.layer * d.n_seq + sq[k]) * d.nkv + g;
      float *dst = (is_k ? e.kv.k : e.kv.v) + (blk * d.n_ctx + ps[k]) * (size_t)hd + jd;
      *(f4 *)dst = x;
      *(f4 *)(dst + half) = y;
      if (is_k) {
        _Float16 *d16 = e.kv.k16 + blk * (size_t)e.kv.ldp * hd + (size_t)ps[k] * hd + jd;
        *(h4 *)d16 = (h4){(_Float16)x.x, (_Float16)x.y, (_Float16)x.z, (_Float16)x.w};
        *(h4 *)(d16 + half) = (h4){(_Float16)y.x, (_Float16)y.y, (_Float16)y.z, (_Float16)y.w};
      }
    }
  }
  // pass 2: the V columns of the tile (a suffix: V heads come last)
  const int v0 = (d.nh + d.nkv) * hd;
  const int cv0 = max(0, min(BNT, v0 - n0));
  const int nv = (min(BNT, N - n0) - cv0) * BMT;  // (column, row) items, rows fastest
  for (int base = 0; base < nv; base += 8 * NT) {
    int mv[8];
    bool okv[8];
    unsigned pv[8], sv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int item = base + tid + NT * u;
      const int r = item % BMT;
      okv[u] = item < nv && m0 + r < M;
      mv[u] = min(m0 + r, M - 1);
      pv[u] = (unsigned)e.rows.pos[mv[u]];
      sv[u] = (unsigned)e.rows.seq[mv[u]];
    }
    pin_regs(pv);
    pin_regs(sv);
    _Float16 hv[8];
    _Float16 *dv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int item = base + tid + NT * u;
      const int r = item % BMT, c = cv0 + min(item / BMT, BNT - 1 - cv0);
      const int n = n0 + c;
      const int head = n / hd, cl = n - head * hd;
      const int dim = (cl >> 1) + (cl & 1) * half;  // natural dim of packed column cl
      const size_t blk = ((size_t)e.layer * d.n_seq + sv[u]) * d.nkv + (size_t)(head - d.nh - d.nkv);
      hv[u] = (_Float16)(T[qkv_tile_idx<BNT>(r, c)] + e.bias[n]);
      dv[u] = e.kv.v16t + blk * (size_t)e.kv.ldp * hd + (size_t)dim * e.kv.ldp + pv[u];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (okv[u]) *dv[u] = hv[u];
  }
}

// ------------------------------------------------------- large-M projections
// Prefill GEMMs with many rows (M >= kBigM) are MFMA-bound.  Block tile
// BM x BN x 64 with NW wavefronts, WGM along M by NW/WGM along N, each owning
// one (BM/WGM) x (BN*WGM/NW) piece of the output as 32 x 32 MFMA tiles.  Both
// operands' 64-wide K slices live in LDS twice (double buffer), so one
// barrier per K slice suffices:
//   write slice t+1 (already in registers) to the free buffer, issue the
//   global loads of slice t+2, multiply slice t, barrier.
// LDS rows are 64 halves (128 B) without padding; 16-byte chunk c of row r
// is stored at chunk c ^ ((r >> 1) & 7).  A 16-byte-per-lane LDS access is
// served 16 lanes (256 B, the 64 banks) at a time, and the 16 consecutive
// rows of an MFMA operand read (or the 2 rows x 8 chunks of a tile write)
// then cover 16 distinct 16-byte bank groups.  Rows past M or N are clamped
// to a valid row and their results are never stored.
constexpr int kBK2 = 64;
constexpr int kBigM = 512;

template <int EPI, int BMT, int BNT, int WGM, int FB = 1, int NW = 4, int S = 1>
__global__ __launch_bounds__(64 * NW) void k_gemm_big(GemmP p) {
  constexpr int NT = 64 * NW;                      // threads
  constexpr int WGN = NW / WGM;                    // wavefronts along M x along N
  constexpr int WTM = BMT / WGM, WTN = BNT / WGN;  // wave tile
  constexpr int TM = WTM / 32, TN = WTN / 32;      // MFMA tiles per wave
  constexpr int RS = NT / 8;                       // rows a loader pass covers
  constexpr int CA = BMT / RS, CB = BNT / RS;      // 16-byte chunks per thread per slice
  static_assert(TM >= 1 && TN >= 1 && CB >= 1, "tile shape");
  __shared__ __attribute__((aligned(16))) _Float16 sAB[2 * (BMT + BNT) * kBK2];
  _Float16 *const sA = sAB;
  _Float16 *const sB = sAB + 2 * BMT * kBK2;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int hi = lane >> 5, l32 = lane & 31;
  const int M = p.M, N = p.N, K = p.K;

  // Tile order.  Blocks are dealt round-robin over the 8 XCDs; XCD x takes
  // the x-th eighth of the row bands, and walks them in groups of G bands,
  // N tiles outermost and the group's bands innermost, so the ~32 blocks an
  // XCD runs at once share G A bands and 32 / G weight tiles in its L2
  // (rather than one A band and 32 weight tiles: 0.5B 4096-row gate/up and
  // down about 3 % faster).  Other grids: consecutive blocks of one XCD walk
  // the N tiles of one row band.
  const int gx = gridDim.x, gy = gridDim.y;
  const int nb = gx * gy;
  const int bid = blockIdx.y * gx + blockIdx.x;
  int tm, tn;
  if ((gy & 7) == 0) {
    const int xcd = bid & 7, t = bid >> 3, bpx = gy >> 3;
    const int G = bpx % 4 == 0 ? 4 : bpx % 3 == 0 ? 3 : bpx % 2 == 0 ? 2 : 1;
    const int grp = t / (G * gx), r = t - grp * (G * gx);
    tm = xcd * bpx + grp * G + r % G;
    tn = r / G;
  } else {
    int tile = bid;
    if ((nb & 7) == 0) tile = (bid & 7) * (nb >> 3) + (bid >> 3);
    tm = tile / gx;
    tn = tile % gx;
  }
  const int m0 = tm * BMT, n0 = tn * BNT;

  // global -> register staging: thread t moves chunk (t & 7) of rows (t >> 3) + RS i
  const int cc = tid & 7, r0 = tid >> 3;
  const _Float16 *Ag[CA];
  const _Float16 *Bg[CB];
#pragma unroll
  for (int i = 0; i < CA; ++i) {
    const int m = min(m0 + r0 + RS * i, M - 1);
    Ag[i] = p.A + (size_t)m * p.lda + cc * 8;
  }
#pragma unroll
  for (int i = 0; i < CB; ++i) {
    const int n = min(n0 + r0 + RS * i, N - 1);
    Bg[i] = p.W + (size_t)n * K + cc * 8;
  }
  // this block's K slices (split-K: blockIdx.z takes p.k_steps of them)
  const int kz0 = blockIdx.z * p.k_steps;
  const int nk = min(K / kBK2 - kz0, p.k_steps);
  auto gload = [&](h8 (&ra)[CA], h8 (&rb)[CB], int kt) {
    const int ko = (kz0 + kt) * kBK2;
#pragma unroll
    for (int i = 0; i < CA; ++i) ra[i] = *(const h8 *)(Ag[i] + ko);
#pragma unroll
    for (int i = 0; i < CB; ++i) rb[i] = *(const h8 *)(Bg[i] + ko);
  };
  auto swrite = [&](int buf, const h8 (&ra)[CA], const h8 (&rb)[CB]) {
    _Float16 *a = sA + buf * BMT * kBK2;
    _Float16 *b = sB + buf * BNT * kBK2;
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int r = r0 + RS * i;
      *(h8 *)(a + r * kBK2 + ((cc ^ ((r >> 1) & 7)) << 3)) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const int r = r0 + RS * i;
      *(h8 *)(b + r * kBK2 + ((cc ^ ((r >> 1) & 7)) << 3)) = rb[i];
    }
  };

  f16x acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // multiplies one 64-wide K slice out of LDS buffer buf: four 16-wide MFMA
  // steps; with FB the operand fragments of step ks+1 are read from LDS
  // before the MFMAs of step ks are issued
  auto frag = [&](const _Float16 *a, const _Float16 *b, int ks, h8 (&af)[TM], h8 (&bf)[TN]) {
    const int ch = ks * 2 + hi;  // logical 16-byte chunk of this lane's operand
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r = wm * WTM + i * 32 + l32;
      af[i] = *(const h8 *)(a + r * kBK2 + ((ch ^ ((r >> 1) & 7)) << 3));
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int r = wn * WTN + j * 32 + l32;
      bf[j] = *(const h8 *)(b + r * kBK2 + ((ch ^ ((r >> 1) & 7)) << 3));
    }
  };
  auto mfma = [&](const h8 (&af)[TM], const h8 (&bf)[TN]) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
  };
  auto compute = [&](int buf) {
    const _Float16 *a = sA + buf * BMT * kBK2;
    const _Float16 *b = sB + buf * BNT * kBK2;
    if (FB) {
      h8 af0[TM], bf0[TN], af1[TM], bf1[TN];
      frag(a, b, 0, af0, bf0);
      frag(a, b, 1, af1, bf1);
      mfma(af0, bf0);
      frag(a, b, 2, af0, bf0);
      mfma(af1, bf1);
      frag(a, b, 3, af1, bf1);
      mfma(af0, bf0);
      mfma(af1, bf1);
    } else {
#pragma unroll
      for (int ks = 0; ks < kBK2 / 16; ++ks) {
        h8 af[TM], bf[TN];
        frag(a, b, ks, af, bf);
        mfma(af, bf);
      }
    }
  };

  if constexpr (S == 1) {
    // Slice kt+1 sits in registers until it is written to LDS buffer
    // (kt+1) & 1; one iteration writes it, requests slice kt+2, multiplies
    // slice kt and ends on the barrier.
    h8 ra[CA], rb[CB];
    gload(ra, rb, 0);
    swrite(0, ra, rb);
    if (nk > 1) gload(ra, rb, 1);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int buf = kt & 1;
      if (kt + 1 < nk) swrite(buf ^ 1, ra, rb);  // its buffer was last read in kt - 1
      if (kt + 2 < nk) gload(ra, rb, kt + 2);
      compute(buf);
      __syncthreads();
    }
  } else {
    // Ring of S register sets: slices kt+1 .. kt+S-1 are in flight while
    // slice kt is multiplied.  An iteration writes slice kt (its loads were
    // issued S iterations earlier) to LDS buffer kt & 1, whose last reader
    // was iteration kt - 2 (behind the barrier of kt - 1), requests slice
    // kt + S into the freed register set, and multiplies slice kt.  Every
    // iteration issues the same loads (past the last slice they re-read it,
    // and the padding iterations multiply nothing), so the compiler's count
    // of outstanding loads stays exact and each LDS write waits only for
    // its own slice rather than draining the ring.
    // (The scheduling barriers keep the sets' loads in issue order: sets
    // issued out of order in the prologue would make the count at the loop
    // head a full drain.)
    h8 ra[S][CA], rb[S][CB];
#pragma unroll
    for (int s = 0; s < S; ++s) {
      gload(ra[s], rb[s], min(s, nk - 1));
      __builtin_amdgcn_sched_barrier(0);
    }
    for (int kb = 0; kb < nk; kb += S) {
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const int kt = kb + s;
        swrite(kt & 1, ra[s], rb[s]);
        __syncthreads();
        gload(ra[s], rb[s], min(kt + S, nk - 1));
        __builtin_amdgcn_sched_barrier(0);
        if (kt < nk) compute(kt & 1);  // (uniform across the block)
      }
    }
  }

  if constexpr (EPI == G_QKV && BMT * BNT <= (BMT + BNT) * kBK2) {
    // the block tile goes through LDS (the operand buffers, free after the
    // last barrier), so the RoPE / KV-store stores are 16-byte row pieces
    // and the transposed binary16 V mirror is written along positions
    float *T = (float *)sAB;
    __syncthreads();  // (every wavefront is past its last operand read)
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wm * WTM + i * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
          T[qkv_tile_idx<BNT>(row, wn * WTN + j * 32 + l32)] = acc[i][j][r];
        }
    __syncthreads();
    qkv_epilogue_lds<BMT, BNT, NT>(p, T, m0, n0);
  } else if constexpr (EPI == G_SWIGLU && BMT >= 128) {
    // the block's SwiGLU outputs (BMT x BNT / 2 halves) go through LDS (the
    // operand buffers, free after the last barrier), so the stores are
    // 16-byte row pieces instead of each lane's 16 single halves down a
    // column (gate/up of 128 and 4096 rows -3 %; with 64-row tiles the two
    // extra barriers cost more than the stores gain)
    _Float16 *T = sAB;  // [BMT][BNT / 2]
    static_assert(BMT * BNT / 2 <= 2 * (BMT + BNT) * kBK2, "output tile fits the operand buffers");
    __syncthreads();  // (every wavefront is past its last operand read)
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float a = acc[i][j][r];
          const float b = __shfl_xor(a, 1, 64);  // (the pair partner: column + 1)
          const int row = wm * WTM + i * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
          const int col = wn * WTN + j * 32 + l32;
          if ((col & 1) == 0) T[row * (BNT / 2) + (col >> 1)] = (_Float16)(silu(a) * b);
        }
    __syncthreads();
    constexpr int CPR = BNT / 16;  // 16-byte pieces of an output row
#pragma unroll
    for (int idx = tid; idx < BMT * CPR; idx += NT) {
      const int row = idx / CPR, ch = idx - row * CPR;
      const int m = m0 + row, col = (n0 >> 1) + ch * 8;
      if (m < M && col < (N >> 1)) *(h8 *)(p.a16 + (size_t)m * p.ld_a + col) = *(const h8 *)(T + row * (BNT / 2) + ch * 8);
    }
  } else {
    // epilogue, one 32 x 32 tile at a time
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        tile_epilogue<EPI>(p, acc[i][j], m0 + wm * WTM + i * 32, n0 + wn * WTN + j * 32 + l32);
  }
}

// ------------------------------------------------- large-M, MFMA-bound core
// 256 x 256 block tile, four wavefronts in a 2 x 2 arrangement, each owning
// 128 x 128 of the output as 4 x 4 MFMA tiles (256 accumulators per lane,
// held in the accumulation registers).  Per 64-wide K slice a wavefront
// reads 32 KB of operand fragments from LDS for 64 MFMAs, a third of what
// the 128 x 128 tile with eight wavefronts reads per MFMA.
// The operand slices go from global memory straight into LDS
// (global_load_lds_dwordx4: lane i's 16 bytes land at byte 16 i of the
// instruction's 1 KB destination), in two stages.  The LDS layout is the
// one of k_gemm_big (chunk slot s of row r holds logical chunk
// s ^ ((r >> 1) & 7)); as the destination of a lane is fixed, the swizzle is
// applied on the source side: each lane loads the logical chunk its slot
// holds.  The loads are counted by vmcnt like any global load; the waits
// for them are explicit.
// Tile order: the grid is 1-D over tiles numbered with M fastest; blocks are
// dealt round-robin over the 8 XCDs, and XCD x takes the x-th contiguous
// eighth of that order, so each XCD streams a band of weight columns once
// while the activations (a few MB) are read by every XCD.
constexpr int kXT = 256;

// s_waitcnt vmcnt(N) with expcnt and lgkmcnt at their maxima (no wait)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// 16 bytes per lane from base + voff into LDS at byte lds + 16 * lane.
// Written as asm: the compiler models this load as a possible LDS access
// of unknown order and then turns every LDS-read wait behind it into
// lgkmcnt(0), which would also wait for the fragment reads just issued.
// The hardware counts it in vmcnt only; the waits for it are explicit.  (An
// M0 write needs one wait state before the load that reads it.)
__device__ __forceinline__ void lds_dma16(const void *base, unsigned voff, unsigned lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(base), "s"(lds)
               : "memory", "m0");
}

// BK: K slice width (32 or 64), NST: LDS stages (NST - 1 slices in flight).
template <int EPI, int BK, int NST>
__global__ __launch_bounds__(256) void k_gemm_xl(GemmP p) {
  constexpr int CPR = BK / 8;         // 16-byte chunks per tile row
  constexpr int RPI = 64 / CPR;       // tile rows one 1 KB load instruction fills
  constexpr int LPO = kXT / RPI / 4;  // load instructions per wavefront per operand
  constexpr int LPT = 2 * LPO;        // ... per slice
  constexpr int KS = BK / 16;         // MFMA steps per slice
  constexpr int SA = kXT * BK;        // halves of one operand slice
  constexpr int SST = 2 * SA;         // halves of one stage
  static_assert(KS % 2 == 0 && LPT <= 16, "slice shape");
  // Bank spread: a 16-byte LDS access serves 16 lanes (256 B, the 64 banks)
  // at a time; rows r .. r + 15 at one logical chunk must land in 16
  // distinct 16-byte bank groups.  256 B hold 16 / CPR rows, so chunk slot
  // s of row r holds logical chunk s ^ ((r / (16 / CPR)) % CPR).
  auto swz = [](int r) { return (r / (16 / CPR)) & (CPR - 1); };
  __shared__ __attribute__((aligned(1024))) _Float16 sm[NST * SST];  // [stage][A | W][row][BK]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int hi = lane >> 5, l32 = lane & 31;
  const int M = p.M, N = p.N, K = p.K;

  const int MB = (M + kXT - 1) / kXT;
  const int nb = gridDim.x, bid = blockIdx.x;
  int tile = bid;
  if ((nb & 7) == 0) tile = (bid & 7) * (nb >> 3) + (bid >> 3);
  const int m0 = (tile % MB) * kXT, n0 = (tile / MB) * kXT;

  // load instruction j of wavefront w fills tile rows RPI (LPO w + j) .. +RPI
  unsigned offA[LPO], offB[LPO];
#pragma unroll
  for (int j = 0; j < LPO; ++j) {
    const int r = RPI * (LPO * wave + j) + lane / CPR;
    const int c = (lane % CPR) ^ swz(r);
    offA[j] = ((unsigned)min(m0 + r, M - 1) * (unsigned)p.lda + 8u * c) * 2u;
    offB[j] = ((unsigned)min(n0 + r, N - 1) * (unsigned)K + 8u * c) * 2u;
  }
  const int kz0 = blockIdx.z * p.k_steps;  // split K: blockIdx.z takes p.k_steps slices
  const int nk = min(K / BK - kz0, p.k_steps);
  const char *Ab = (const char *)p.A + (size_t)kz0 * BK * 2;
  const char *Wb = (const char *)p.W + (size_t)kz0 * BK * 2;
  // load q (A rows, then W rows) of slice kt (clamped: the padding requests
  // past the end re-read the last slice, so every iteration issues the same
  // loads) into stage st
  const unsigned lds0 = (unsigned)(size_t)(__attribute__((address_space(3))) _Float16 *)sm;
  auto gload = [&](int q, int kt, int st) {
    const unsigned ko = (unsigned)min(kt, nk - 1) * (BK * 2);
    const unsigned dst =
        lds0 + 2u * (st * SST + (q < LPO ? 0 : SA) + (wave * LPO + (q % LPO)) * 512);
    lds_dma16(q < LPO ? Ab + ko : Wb + ko, q < LPO ? offA[q] : offB[q - LPO], dst);
  };

  // fragment reads: rows wm * 128 + 32 i + l32 of A and wn * 128 + 32 j + l32
  // of W (their swizzle depends on l32 only), logical chunk 2 ks + hi of the
  // 16-wide step ks
  const int f = swz(l32);
  const int ra = (wm * 128 + l32) * BK, rb = (wn * 128 + l32) * BK;
  auto frag = [&](int st, int ks, h8 (&af)[4], h8 (&bf)[4]) {
    const int co = ((2 * ks + hi) ^ f) << 3;
    const _Float16 *a = sm + st * SST + ra + co;
    const _Float16 *b = sm + st * SST + SA + rb + co;
#pragma unroll
    for (int i = 0; i < 4; ++i) af[i] = *(const h8 *)(a + i * 32 * BK);
#pragma unroll
    for (int j = 0; j < 4; ++j) bf[j] = *(const h8 *)(b + j * 32 * BK);
  };
  f16x acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  // the 16 MFMAs of one step; with LD, load q of slice kt_ld goes out after
  // MFMA q, pinned there (the address arithmetic and issue overlap the
  // matrix pipe; left to the scheduler, the loads bunch up behind the first
  // few MFMAs and the rest of the step's MFMAs wait behind their issue)
  auto mfma = [&](const h8 (&af)[4], const h8 (&bf)[4], bool LD, int kt_ld, int st_ld) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      acc[q >> 2][q & 3] =
          __builtin_amdgcn_mfma_f32_32x32x16_f16(af[q >> 2], bf[q & 3], acc[q >> 2][q & 3], 0, 0, 0);
      if (LD && q < LPT) {
        gload(q, kt_ld, st_ld);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  // (program order is kept: each phase's LDS reads must be in flight while
  // the previous phase's MFMAs run, which the scheduler would not arrange)
#define XL_PHASE __builtin_amdgcn_sched_barrier(0)

  // Iteration kt multiplies slice kt (stage kt % NST).  The fragments of
  // step s + 1 are read while step s is multiplied.  Before its last step it
  // waits for its own loads of slice kt + 1 (the NST - 2 newer slices may
  // stay in flight), meets the barrier (everyone's loads of slice kt + 1
  // have landed, and everyone's reads of slice kt are done) and reads slice
  // kt + 1's first step; its last step's MFMAs, whose fragments are already
  // in registers, then carry the requests of slice kt + NST into the stage
  // slice kt has just left.  A request thus goes out a step earlier than it
  // could from the next iteration's first step (hd-128 gate/up 15.5 -> 14.7
  // ms, down 7.6 -> 7.0 ms per 2048-token prefill).  Requests past the last
  // slice re-read it, so every iteration issues the same loads and the wait
  // counts stay exact; the kernel drains them before its epilogue.
  h8 a0[4], b0[4], a1[4], b1[4];
#pragma unroll
  for (int s = 0; s < NST; ++s)
#pragma unroll
    for (int q = 0; q < LPT; ++q) gload(q, s, s);
  wait_vmcnt<(NST - 1) * LPT>();
  __syncthreads();
  frag(0, 0, a0, b0);
  int cur = 0, nxt = 1;  // stages of slices kt and kt + 1
  for (int kt = 0; kt < nk; ++kt) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      XL_PHASE;
      if (ks + 1 < KS) {
        if (ks & 1)
          frag(cur, ks + 1, a0, b0);
        else
          frag(cur, ks + 1, a1, b1);
      } else {
        wait_vmcnt<(NST - 2) * LPT>();
        __syncthreads();
        XL_PHASE;
        frag(nxt, 0, a0, b0);
      }
      XL_PHASE;
      if (ks & 1)
        mfma(a1, b1, ks == KS - 1, kt + NST, cur);
      else
        mfma(a0, b0, false, 0, 0);
    }
    cur = nxt;
    nxt = nxt + 1 == NST ? 0 : nxt + 1;
  }
  wait_vmcnt<0>();  // (the requests past the last slice land before the block may end)
  XL_PHASE;

  // One 32 x 32 tile at a time, its sums copied out of the accumulation
  // registers right before use (the copies are explicit: left to the
  // compiler, all 256 are made at the loop exit, which needs more
  // registers than there are and spills them to scratch).
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f16x v;
#pragma unroll
      for (int r = 0; r < 16; ++r) asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v[r]) : "a"(acc[i][j][r]));
      tile_epilogue<EPI>(p, v, m0 + wm * 128 + i * 32, n0 + wn * 128 + j * 32 + l32);
      XL_PHASE;
    }
#undef XL_PHASE
}

template <int EPI, int BMT, int BNT, int WGM, int FB = 0, int NW = 4, int S = 1>
static void launch_big(GemmP p, int splits, hipStream_t st) {
  const int nk = p.K / kBK2;
  p.k_steps = (nk + splits - 1) / splits;
  splits = (nk + p.k_steps - 1) / p.k_steps;
  if (splits <= 1) p.ws = nullptr;
  dim3 grid((p.N + BNT - 1) / BNT, (p.M + BMT - 1) / BMT, splits);
  hipLaunchKernelGGL((k_gemm_big<EPI, BMT, BNT, WGM, FB, NW, S>), grid, dim3(64 * NW), 0, st, p);
}

// Large-M GEMM with long K (>= 2048, M >= 1024), residual and SwiGLU
// epilogues: k_gemm_xl.  Measured against the best k_gemm_big tile on the
// hd-128 shapes: gate/up 2048 x 37888 x 3584 635 -> 572 us, down
// 2048 x 3584 x 18944 (split in two) 351 -> 271 us, WO 2048 x 3584 x 3584
// (two splits) 71 -> 63 us.  Residual GEMMs with fewer tiles than CUs split
// K so that about 256 blocks run; their partial sums go to the workspace
// (at most 256 / tiles sets of M x N, i.e. <= 64 MB) and are folded in by
// the next RMSNorm.  Returns the number of pending partial-sum sets (0:
// applied).
template <int EPI>
static int launch_xl(GemmP p, const Workspace &wsp, hipStream_t st) {
  constexpr int BK = 64;
  const int nk = p.K / BK;
  const int tiles = ((p.M + kXT - 1) / kXT) * ((p.N + kXT - 1) / kXT);
  int splits = 1;
  if (EPI == G_RESID && wsp.buf && tiles < 256) {
    splits = min(256 / tiles, min(kMaxSplits, nk));
    splits = min(splits, (int)(wsp.bytes / ((size_t)p.M * p.N * 4)));
    if (splits < 1) splits = 1;
  }
  p.k_steps = (nk + splits - 1) / splits;
  splits = (nk + p.k_steps - 1) / p.k_steps;
  p.ws = splits > 1 ? wsp.buf : nullptr;
  hipLaunchKernelGGL((k_gemm_xl<EPI, BK, 2>), dim3(tiles, 1, splits), dim3(256), 0, st, p);
  return splits > 1 ? splits : 0;
}

// Tile of the other large-M GEMMs (all with 8 wavefronts, 2 along M x 4
// along N).  Short K (< 2048, the 0.5B shape's 896): 128 x 128 (measured
// 381-643 TFLOP/s on the 4096-row 0.5B projections, against 304-590 with 4
// wavefronts).  Long K: the tile whose measured per-CU rate times the number
// of rounds of blocks over the 256 CUs is cheapest, among 256 x 256 (910
// TFLOP/s on a 2048 x 37888 x 3584 GEMM), 128 x 256 (850) and 128 x 128 (740).
// A residual GEMM on 128 x 128 tiles whose tiles cannot fill the CUs
// (fewer than 192) splits K so that about 256 blocks run, the partial sums
// pending in the workspace for the next RMSNorm (as launch_xl; 1.5B head
// layout, 512 rows, down 1536 x 8960: 48 tiles).  Returns the pending
// split count (0: applied).
template <int EPI>
static int launch_big_resid(GemmP p, const Workspace &wsp, hipStream_t st) {
  int splits = 1;
  const int nk = p.K / kBK2;
  const int tiles = ((p.M + 127) / 128) * ((p.N + 127) / 128);
  if (EPI == G_RESID && wsp.buf && tiles < 192) {
    splits = min(256 / tiles, min(kMaxSplits, nk));
    splits = min(splits, (int)(wsp.bytes / ((size_t)p.M * p.N * 4)));
    if (splits < 1) splits = 1;
  }
  p.ws = splits > 1 ? wsp.buf : nullptr;
  p.atomic_out = 0;
  const int ks = (nk + splits - 1) / splits;
  const int used = (nk + ks - 1) / ks;
  launch_big<EPI, 128, 128, 2, 0, 8>(p, splits, st);
  return used > 1 ? used : 0;
}

template <int EPI>
static int launch_large_m(const GemmP &p, const Workspace &wsp, hipStream_t st) {
  if constexpr (EPI == G_QKV) {
    // (its LDS-staged epilogue fits tiles up to 128 x 128) Rows per tile:
    // the one of 128, 64 and 32 with the least rounds of blocks over the 256
    // CUs times rows per tile over the rate a row of that tile reaches
    // (relative rates 1, 0.83, 0.59, measured on the hd-128 2048-row QKV).
    // Measured: 0.5B 4096 rows (288 tiles of 128): 0.78 -> 0.67 ms per
    // prefill on 64-row tiles; 1.5B head layout, 512 rows x 2048 (64 tiles
    // of 128): 0.86 -> 0.66 ms on 32-row tiles; hd-128 2048 rows stays on
    // 128 (32-row tiles: 3.36 -> 4.29 ms).  With long K (>= 2048) the
    // 128-row tiles keep two K slices in flight in register sets (hd-128
    // 2048-row QKV 3.30 -> 3.19 ms per prefill; three sets 3.29; at K = 896
    // the ring was slower).
    const int nt = (p.N + 127) / 128;
    const int rows[3] = {128, 64, 32};
    const double rate[3] = {1.0, 0.83, 0.59};
    int best = 0;
    double best_cost = 1e300;
    for (int i = 0; i < 3; ++i) {
      const long tiles = (long)((p.M + rows[i] - 1) / rows[i]) * nt;
      const double cost = (double)((tiles + 255) / 256) * rows[i] / rate[i];
      if (cost < best_cost * 0.98) {
        best_cost = cost;
        best = i;
      }
    }
    if (best == 0 && p.K >= 2048)
      launch_big<EPI, 128, 128, 2, 0, 8, 2>(p, 1, st);
    else if (best == 0)
      launch_big<EPI, 128, 128, 2, 0, 8>(p, 1, st);
    else if (best == 1)
      launch_big<EPI, 64, 128, 2, 0, 8>(p, 1, st);
    else
      launch_big<EPI, 32, 128, 1, 0, 4>(p, 1, st);
    return 0;
  } else {
    // (residual GEMMs with fewer than 96 tiles would need more than two
    // partial-sum sets, whose folding costs the next RMSNorm more than the
    // split saves: 0.5B down)
    const int tiles = ((p.M + kXT - 1) / kXT) * ((p.N + kXT - 1) / kXT);
    if (p.K >= 2048 && p.M >= 1024 && (EPI == G_SWIGLU || tiles >= 96))
      return launch_xl<EPI>(p, wsp, st);
  }
  if (p.K < 2048 || (EPI == G_RESID && ((p.M + 127) / 128) * ((p.N + 127) / 128) < 192))
    return launch_big_resid<EPI>(p, wsp, st);
  struct Cand { int bm, bn; double rate; };
  const Cand cand[3] = {{256, 256, 910.0}, {128, 256, 850.0}, {128, 128, 740.0}};
  int best = 2;
  double best_cost = 1e300;
  for (int i = 0; i < 3; ++i) {
    const long tiles = (long)((p.M + cand[i].bm - 1) / cand[i].bm) * ((p.N + cand[i].bn - 1) / cand[i].bn);
    const double cost = (double)((tiles + 255) / 256) * cand[i].bm * cand[i].bn / cand[i].rate;
    if (cost < best_cost) {
      best_cost = cost;
      best = i;
    }
  }
  if (best == 0)
    launch_big<EPI, 256, 256, 2, 1, 8>(p, 1, st);
  else if (best == 1)
    launch_big<EPI, 128, 256, 2, 1, 8>(p, 1, st);
  else
    launch_big<EPI, 128, 128, 2, 0, 8>(p, 1, st);
  return 0;
}

// ------------------------------------------------------ skinny projections
// Fewer rows (8 < M < kBigM): weight streaming and latency dominate.  Block
// tile (32 TM) x 32 with the four wavefronts splitting the block's K range
// (wave w takes a contiguous quarter of the 16-wide MFMA steps).  Operands
// are read straight from global memory into MFMA registers (every weight
// and activation element is used by exactly one wavefront of the block, so
// LDS staging would not save a load); U steps of loads are kept in flight.
// One load instruction covers 32 B of each of 32 rows, so the loads are
// cached: the following steps of the same wavefront read the rest of each
// 128-byte line from the cache instead of HBM.
// The four partial tiles are summed through LDS, wavefront t finishing
// tile t.  A block may also take only a share of K (split-K, residual
// GEMMs only: raw partial sums, folded in by the next RMSNorm).
template <int EPI, int TM, int NWS = 4, bool NORM = false>
__global__ __launch_bounds__(64 * NWS) void k_gemm_skinny(GemmP p) {
  constexpr int U = TM >= 4 ? 4 : 8;  // MFMA steps of loads in flight per wavefront
  static_assert(!NORM || (EPI == G_QKV && TM == 1 && NWS == 8), "fused RMSNorm: QKV, 32 rows");
  __shared__ f16x sRed[NWS][TM][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hi = lane >> 5, l32 = lane & 31;
  const int M = p.M, N = p.N, K = p.K;
  const int m0 = blockIdx.y * 32 * TM, n0 = blockIdx.x * 32;

  // K steps of this block, then of this wavefront
  const int steps = K / 16;
  const int bs0 = blockIdx.z * p.k_steps, bs1 = min(steps, bs0 + p.k_steps);
  const int per = (bs1 - bs0 + NWS - 1) / NWS;
  const int s0 = bs0 + wave * per, s1 = min(bs1, s0 + per);

  const _Float16 *Ap[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i)
    Ap[i] = p.A + (size_t)min(m0 + i * 32 + l32, M - 1) * p.lda + hi * 8;
  const _Float16 *Bp = p.W + (size_t)min(n0 + l32, N - 1) * K + hi * 8;

  f16x acc[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;

  // Fused RMSNorm (K <= 1024: at most U steps per wavefront).  Every load of
  // the wavefront goes out at once: its steps of the f32 residual row and of
  // the weights, and the block stages the norm gains in LDS.  The row's sum
  // of squares is then reduced over the two lane halves and the wavefronts,
  // and the normed, gained values become the binary16 A fragments, as the
  // separate RMSNorm kernel would have written them.
  __shared__ float sSS[NORM ? NWS : 1][32];
  __shared__ __attribute__((aligned(16))) float sG[NORM ? 1024 : 4];
  if constexpr (NORM) {
    const float *Hp = p.hx + (size_t)min(m0 + l32, M - 1) * p.ldhx + hi * 8;
    f4 hv[U][2];
    h8 bf[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // (steps past s1 repeat its last, unused; a wavefront without steps
      // reads step 0)
      const int k = max(min(s0 + u, s1 - 1), 0) * 16;
      hv[u][0] = *(const f4 *)(Hp + k);
      hv[u][1] = *(const f4 *)(Hp + k + 4);
      bf[u] = *(const h8 *)(Bp + k);
    }
    for (int k = tid * 4; k < K; k += 64 * NWS * 4) *(f4 *)(sG + k) = *(const f4 *)(p.gain + k);
    float ss = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (s0 + u < s1)
#pragma unroll
        for (int c = 0; c < 2; ++c)
          ss += hv[u][c].x * hv[u][c].x + hv[u][c].y * hv[u][c].y + hv[u][c].z * hv[u][c].z +
                hv[u][c].w * hv[u][c].w;
    ss += __shfl_xor(ss, 32, 64);
    if (hi == 0) sSS[wave][l32] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < NWS; ++w) tot += sSS[w][l32];
    const float inv = 1.0f / sqrtf(tot / (float)K + p.eps);
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (s0 + u < s1) {
        const int k = (s0 + u) * 16 + hi * 8;
        const f4 g0 = *(const f4 *)(sG + k), g1 = *(const f4 *)(sG + k + 4);
        const f4 x0 = hv[u][0] * inv * g0, x1 = hv[u][1] * inv * g1;
        const h8 af = {(_Float16)x0.x, (_Float16)x0.y, (_Float16)x0.z, (_Float16)x0.w,
                       (_Float16)x1.x, (_Float16)x1.y, (_Float16)x1.z, (_Float16)x1.w};
        acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, bf[u], acc[0], 0, 0, 0);
      }
  }

  for (int s = s0; s < (NORM ? s0 : s1); s += U) {
    h8 af[U][TM], bf[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = min(s + u, s1 - 1) * 16;  // (a step past s1 repeats the last, unused)
      bf[u] = *(const h8 *)(Bp + k);  // (cached: the next steps read the rest of each line)
#pragma unroll
      for (int i = 0; i < TM; ++i) af[u][i] = *(const h8 *)(Ap[i] + k);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (s + u < s1)
#pragma unroll
        for (int i = 0; i < TM; ++i)
          acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[u][i], bf[u], acc[i], 0, 0, 0);
  }
  // The partial sums go to LDS as [wavefront][row tile][accumulator row]
  // [lane], so every read below (one accumulator row across the lanes)
  // falls on consecutive banks; stored as one 64-byte vector per lane, the
  // same reads were 16-way bank conflicts (QKV: 1.8 us for its eight
  // wavefronts; in the residual GEMMs, where one to four wavefronts read,
  // the conflicts took 3/4 of the LDS time but no measurable kernel time).
  float *const sT = (float *)sRed;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) sT[((wave * TM + i) * 16 + r) * 64 + lane] = acc[i][r];
  __syncthreads();
  if constexpr (EPI == G_QKV && TM == 1 && NWS == 8) {
    // every wavefront finishes two of the tile's 16 accumulator rows, so the
    // RoPE / KV-store epilogue runs on all eight wavefronts
    const int n = n0 + l32;
    int m[2];
    bool ok[2];
    float a[2], b[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int r = 2 * wave + u;
      float x = sT[r * 64 + lane];
#pragma unroll
      for (int w = 1; w < NWS; ++w) x += sT[(w * 16 + r) * 64 + lane];  // (TM = 1)
      a[u] = x;
      b[u] = __shfl_xor(x, 1, 64);  // the pair partner (column n + 1)
      const int mm = m0 + 8 * (r >> 2) + 4 * hi + (r & 3);
      ok[u] = mm < M && n < N && (n & 1) == 0;
      m[u] = min(mm, M - 1);
    }
    qkv_store_rows<2, 2>(p.d, p.qkv, m, min(n & ~1, N - 2), a, b, ok);
    return;
  }
  if (wave >= TM) return;
  f16x v;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float x = sT[(wave * 16 + r) * 64 + lane];
#pragma unroll
    for (int w = 1; w < NWS; ++w) x += sT[((w * TM + wave) * 16 + r) * 64 + lane];
    v[r] = x;
  }

  tile_epilogue<EPI>(p, v, m0 + wave * 32, n0 + l32);
}

// Launch shape of a skinny GEMM: rows per block 32 TM (TM = 4, 2, 1) and,
// for residual GEMMs, K splits (added into h with float atomics); the
// choice minimises the bytes the busiest CU loads (A and W of its blocks),
// with blocks dealt evenly over 256 CUs, plus a charge per split (the extra
// adds).
template <int EPI>
static void skinny_shape(const GemmP &p, const Workspace &wsp, int &best_tm, int &best_sp) {
  const int steps = p.K / 16;
  const int nt = (p.N + 31) / 32;
  best_tm = 1;
  best_sp = 1;
  double best_cost = 1e30;
  for (int tm = 4; tm >= 1; tm >>= 1) {
    const int mt = (p.M + 32 * tm - 1) / (32 * tm);
    const int max_sp = (EPI == G_RESID && wsp.buf) ? kMaxSplits : 1;
    for (int sp = 1; sp <= max_sp; ++sp) {
      if ((size_t)sp * p.M * p.N * 4 > wsp.bytes && sp > 1) break;
      const int ks = (steps + sp - 1) / sp;
      const int blocks = nt * mt * ((steps + ks - 1) / ks);
      const double vol = (32.0 * tm + 32.0) * ks * 16 * 2;
      const double cost = vol * ((blocks + 255) / 256) + (sp > 1 ? sp * 4.0 * p.M * 32 : 0.0);
      if (cost < best_cost * 0.98) {
        best_cost = cost;
        best_tm = tm;
        best_sp = sp;
      }
    }
  }
}

template <int EPI>
static int launch_skinny(GemmP p, const Workspace &wsp, hipStream_t st) {
  const int steps = p.K / 16;
  const int nt = (p.N + 31) / 32;
  int best_tm, best_sp;
  skinny_shape<EPI>(p, wsp, best_tm, best_sp);
  p.k_steps = (steps + best_sp - 1) / best_sp;
  const int splits = (steps + p.k_steps - 1) / p.k_steps;
  p.ws = splits > 1 ? wsp.buf : nullptr;
  p.atomic_out = 1;  // (the split sums go straight into h)
  dim3 grid(nt, (p.M + 32 * best_tm - 1) / (32 * best_tm), splits);
  if (EPI == G_QKV && best_tm == 1) {
    // (no K split across blocks for QKV: eight wavefronts split the block's
    // K range, so each one's share of steps goes out in one batch of loads)
    hipLaunchKernelGGL((k_gemm_skinny<EPI, 1, 8>), grid, dim3(512), 0, st, p);
    return 0;
  }
  switch (best_tm) {
    case 4: hipLaunchKernelGGL((k_gemm_skinny<EPI, 4>), grid, dim3(256), 0, st, p); break;
    case 2: hipLaunchKernelGGL((k_gemm_skinny<EPI, 2>), grid, dim3(256), 0, st, p); break;
    default: hipLaunchKernelGGL((k_gemm_skinny<EPI, 1>), grid, dim3(256), 0, st, p); break;
  }
  return 0;
}

// Mid-M launch (8 < M < kBigM): tile BMT x BNT with NW wavefronts, S K
// slices in flight (k_gemm_big's register ring), FB fragment read-ahead,
// and for residual GEMMs a K split; returns the pending split count (0:
// applied directly).
template <int EPI, int BMT, int BNT, int WGM, int S, int FB = 0, int NW = 4>
static int launch_ring(GemmP p, int splits, const Workspace &wsp, hipStream_t st) {
  const int nk = p.K / kBK2;
  if (EPI != G_RESID || !wsp.buf) splits = 1;
  splits = max(1, min(splits, min(kMaxSplits, nk)));
  while (splits > 1 && (size_t)splits * p.M * p.N * 4 > wsp.bytes) --splits;
  p.ws = splits > 1 ? wsp.buf : nullptr;
  const int ks = (nk + splits - 1) / splits;
  const int used = (nk + ks - 1) / ks;  // launch_big's effective split count
  launch_big<EPI, BMT, BNT, WGM, FB, NW, S>(p, splits, st);
  return used > 1 ? used : 0;
}


// K % 64 == 0.  Many rows: launch_large_m.  Fewer rows: the weights
// dominate and the K loop is latency-bound, so the tiles keep a ring of K
// slices in flight, and long-K residual GEMMs split K over about 256 blocks
// whose sums are added into h atomically (0.5B 128-token prefill 1.24 ->
// 1.20 ms against split sums folded in by the next RMSNorm).  Returns the
// number of split-K partial-sum sets left pending in the workspace (0 when
// the result was applied directly).
template <int EPI>
static int launch_tiles(GemmP p, const Workspace &wsp, hipStream_t st) {
  if (p.M >= kBigM) return launch_large_m<EPI>(p, wsp, st);
  if (p.K <= 1024 && p.N <= 2048) return launch_skinny<EPI>(p, wsp, st);
  // gate/up of up to 128 rows: a ring of K slices in flight and the next
  // step's LDS fragments read ahead (measured on the 0.5B gate/up GEMM: two
  // slices, 64 rows 12.6 -> 9.2 us, 128 rows 13.0 -> 10.9 us; four slices
  // at up to 64 rows, 64-sequence decode step 1.475 -> 1.460 ms, no gain at
  // 128 rows)
  if constexpr (EPI == G_SWIGLU) {
    if (p.M <= 64) return launch_ring<EPI, 64, 64, 2, 4, 1, 4>(p, 1, wsp, st);
    if (p.M <= 128) return launch_ring<EPI, 128, 64, 4, 2, 1, 8>(p, 1, wsp, st);
  }
  const int nk = p.K / kBK2;
  // (up to 64 rows: 64 x 64 tiles, so a block reads no clamped rows and
  // half the activation slice of a 128 x 32 tile per output column)
  const bool m64 = p.M <= 64;
  int splits = 1;
  if (EPI == G_RESID && p.K >= 2048 && wsp.buf) {
    const int blocks = m64 ? (p.N + 63) / 64 : ((p.N + 31) / 32) * ((p.M + 127) / 128);
    splits = max(1, 256 / blocks);
    splits = min(splits, min(kMaxSplits, nk));
    const size_t per = (size_t)p.M * p.N * 4;
    splits = min(splits, (int)(wsp.bytes / per));
    if (splits < 1) splits = 1;
  }
  p.ws = splits > 1 ? wsp.buf : nullptr;
  p.atomic_out = 1;  // (few rows: the split sums go straight into h)
  // (a ring of two K slices in register sets and the fragment read-ahead:
  // 0.5B down at 128 rows 0.286 -> 0.260 ms per prefill, 64-sequence decode
  // step 1.472 -> 1.439 ms; four slices pad the few slices of a K split)
  if (m64)
    launch_big<EPI, 64, 64, 2, 1, 4, 2>(p, splits, st);
  else
    launch_big<EPI, 128, 32, 4, 1, 4, 2>(p, splits, st);
  return 0;
}

// Every projection but the lm_head runs on the tile kernels (K is a
// multiple of 64 for every supported shape: n_embd % 64 == 0 and the FFN
// width is padded to 64).
template <int EPI>
static int launch(GemmP p, const Workspace &wsp, hipStream_t st) {
  return launch_tiles<EPI>(p, wsp, st);
}


static GemmP base(const _Float16 *A, int lda, int M, const uint16_t *W, int N, int K) {
  GemmP p{};
  p.A = A;
  p.lda = lda;
  p.M = M;
  p.W = (const _Float16 *)W;
  p.N = N;
  p.K = K;
  return p;
}

void gemm_qkv(const Dims &d, const LayerW &w, const _Float16 *x, int lda, int M,
              const QkvEpi &e, const Workspace &ws, hipStream_t st) {
  GemmP p = base(x, lda, M, w.wqkv, d.nqkv, d.H);
  p.d = d;
  p.qkv = e;
  launch<G_QKV>(p, ws, st);
}

bool qkv_fuses_norm(const Dims &d, int M, const Workspace &ws) {
  GemmP p = base(nullptr, 0, M, nullptr, d.nqkv, d.H);
  if (M >= kBigM || p.K > 1024 || p.N > 2048) return false;  // (not the skinny kernel)
  int tm, sp;
  skinny_shape<G_QKV>(p, ws, tm, sp);
  return tm == 1;
}

void gemm_qkv_normed(const Dims &d, const LayerW &w, const float *h, int ldh, int M, float eps,
                     const QkvEpi &e, hipStream_t st) {
  GemmP p = base(nullptr, 0, M, w.wqkv, d.nqkv, d.H);
  p.d = d;
  p.qkv = e;
  p.hx = h;
  p.ldhx = ldh;
  p.gain = w.attn_norm;
  p.eps = eps;
  p.k_steps = p.K / 16;
  const dim3 grid((p.N + 31) / 32, (M + 31) / 32, 1);
  hipLaunchKernelGGL((k_gemm_skinny<G_QKV, 1, 8, true>), grid, dim3(512), 0, st, p);
}

int gemm_resid(const uint16_t *W, int N, int K, const _Float16 *x, int lda, int M, float *h,
               int ldh, const Workspace &ws, hipStream_t st) {
  GemmP p = base(x, lda, M, W, N, K);
  p.h = h;
  p.ldh = ldh;
  return launch<G_RESID>(p, ws, st);
}

void gemm_swiglu(const Dims &d, const LayerW &w, const _Float16 *x, int lda, int M,
                 _Float16 *a, int ld_a, const Workspace &ws, hipStream_t st) {
  GemmP p = base(x, lda, M, w.wgu, 2 * d.I_pad, d.H);
  p.a16 = a;
  p.ld_a = ld_a;
  launch<G_SWIGLU>(p, ws, st);
}

void gemm_lmhead(const Dims &d, const uint16_t *W, const _Float16 *x, int lda, int M,
                 const ArgmaxEpi &e, hipStream_t st) {
  GemmP p = base(x, lda, M, W, d.V, d.H);
  p.am = e;
  p.k_steps = d.H / BK;
  // (64-row tiles up to 64 rows: a 128-row tile would load and multiply
  // every A row twice)
  if (M <= 64)
    hipLaunchKernelGGL(k_gemm_lmhead<64>, dim3((d.V + BN - 1) / BN, 1), dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL(k_gemm_lmhead<128>, dim3((d.V + BN - 1) / BN, (M + 127) / 128), dim3(256), 0, st, p);
  argmax_finalize(e, M, st);
}

}  // namespace q2
