// Causal grouped-query attention kernels.
//
// Query head h reads KV head h / group (contiguous groups: on the 0.5B shape
// KV head j serves query heads 7j..7j+6, nnterp Qwen2 page, "Grouped-query
// attention"); scores are scaled by head_dim^-0.5; a row at position p sees
// the KV slots 0..p of its own sequence (full causal attention, no window).
//
// Which kernels share a KV head's K / V across its query group:
//  * k_attn_decode_mfma (chunked decode attention: the group's heads are
//    the columns of its score tile) and k_attn_prefill (MFMA prefill
//    attention: one wavefront per head over K / V tiles staged once in LDS)
//    load each K / V tile once per KV head and use it for every query head
//    of the group (k_attn_prefill's short-prompt form runs one head per
//    block instead, so the group's heads spread over CUs);
//  * k_attn_wo1 and k_attn_wo (attention fused with WO, short contexts) do
//    not: a block serves one (WO row chunk, query head) pair and reads that
//    head's K / V itself.  Their cost is the per-block K / V fetch and the
//    kernel's fixed latency, not the total K / V traffic (see k_attn_wo1).
#include <algorithm>

#include "q2_device.h"

namespace q2 {

// ------------------------------------------------------------------ decode
// Chunked decode attention (k_attn_decode_mfma): one wavefront per (64-key
// chunk, KV head, query row).  A single-chunk call writes the normalised
// output; otherwise every wavefront writes its chunk's (un-normalised
// output, maximum, exp-sum) record and k_attn_merge (or k_merge_wo, which
// also multiplies by WO) combines the records.  No block waits on another.
struct AttnDecP {
  Dims d;
  int layer;
  KVCache kv;
  const float *q;
  int ldq;
  RowInfo rows;
  AttnPartials part;
  float *o32;
  _Float16 *o16;
  int ldo;
  float scale;
};

// One wavefront per (64-key chunk, KV head, query row) on the matrix core,
// reading the binary16 mirror of the cache (K as [pos][d], V transposed as
// [d][pos]) straight into MFMA operands, every load issued before the
// first is used.  The group's query
// heads are the 32 columns of the score tile (columns >= G are zero and
// unused): S[key][head] = K Q^T over 16-wide d steps, then per head (a
// lane's 16 keys of each 32-key half, and its partner lane l ^ 32 holding
// the other 16) the maximum and the base-2 weights, and O^T[d][head] =
// V^T P with the weights' binary16 key order matched by the V^T reads.
// Keys past the row's position are masked (score -inf, V zeroed).  The
// record's maximum is in natural-log units (the merges weight records by
// e^(m_c - M)).
template <int HD, int G, bool DIRECT>
__global__ __launch_bounds__(64) void k_attn_decode_mfma(AttnDecP p) {
  static_assert(kChunkKeys == 64 && G <= 32, "64-key chunks, at most 32 heads per group");
  constexpr int KSTEPS = HD / 16;               // 16-wide d steps of Q K^T
  constexpr int DT = HD >= 32 ? HD / 32 : 1;    // 32-row d tiles of O^T
  constexpr bool LATE_V = HD > 64;              // (wide heads: V after the scores, fewer registers)
  const int lane = threadIdx.x, hi = lane >> 5, l32 = lane & 31;
  const int c = blockIdx.x, g = blockIdx.y, m = blockIdx.z;
  const int pos = p.rows.pos[m];
  const int seq = p.rows.seq[m];
  const int kb = c * kChunkKeys;
  const int nk = min(kChunkKeys, pos + 1 - kb);
  if (nk <= 0) return;  // uniform across the wavefront
  const size_t b16 = p.kv.off16(p.d, p.layer, seq, g);
  const _Float16 *kg = p.kv.k16 + b16 + (size_t)kb * HD;  // (chunk slots stay inside ldp)
  const _Float16 *vg = p.kv.v16t + b16 + kb;
  const int hq = min(l32, G - 1);
  const float *qp = p.q + (size_t)m * p.ldq + (size_t)(g * G + hq) * HD;
  const int vrow = min(l32, HD - 1);  // (d rows HD..31 of a 16-wide head: zeroed below)

  f4 qv[KSTEPS][2];
#pragma unroll
  for (int st = 0; st < KSTEPS; ++st) {
    qv[st][0] = *(const f4 *)(qp + st * 16 + hi * 8);
    qv[st][1] = *(const f4 *)(qp + st * 16 + hi * 8 + 4);
  }
  h8 kf[2][KSTEPS];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int st = 0; st < KSTEPS; ++st)
      kf[hf][st] = *(const h8 *)(kg + (size_t)(hf * 32 + l32) * HD + st * 16 + hi * 8);
  h4 vf[DT][2][4];
  auto vload = [&]() {
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          vf[t][hf][j] = *(const h4 *)(vg + (size_t)(t * 32 + vrow) * p.kv.ldp + hf * 32 + 8 * j + 4 * hi);
  };
  if (!LATE_V) vload();
  __builtin_amdgcn_sched_barrier(0);  // (every load in flight before the first is used)

  // Q operand: column l32 = head g*G + l32, scaled by head_dim^-0.5 log2(e)
  const float qs = l32 < G ? p.scale * 1.4426950408889634f : 0.f;
  h8 qf[KSTEPS];
#pragma unroll
  for (int st = 0; st < KSTEPS; ++st)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      qf[st][j] = (_Float16)(qv[st][0][j] * qs);
      qf[st][4 + j] = (_Float16)(qv[st][1][j] * qs);
    }
  f16x s[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[hf][r] = 0.f;
#pragma unroll
    for (int st = 0; st < KSTEPS; ++st)
      s[hf] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf[hf][st], qf[st], s[hf], 0, 0, 0);
  }
  if (LATE_V) vload();
  if (nk < kChunkKeys) {  // (the row's last chunk; uniform)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (hf * 32 + 8 * (r >> 2) + 4 * hi + (r & 3) >= nk) s[hf][r] = kNegInf;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (hf * 32 + 8 * j + 4 * hi + e >= nk) vf[t][hf][j][e] = (_Float16)0.f;
  }
  if (HD < 32 && l32 >= HD) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int j = 0; j < 4; ++j) vf[0][hf][j] = (h4){0, 0, 0, 0};
  }
  float mx = kNegInf;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[hf][r]);
  mx = max32(mx);  // (key 0 of the chunk is always visible: finite)
  h8 pb[2][2];
  float l = 0.f;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int r = 0; r < 16; ++r) pb[hf][r >> 3][r & 7] = (_Float16)__builtin_amdgcn_exp2f(s[hf][r] - mx);
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int k = 0; k < 8; k += 2)
        l = __builtin_amdgcn_fdot2((h2){pb[hf][j][k], pb[hf][j][k + 1]}, (h2){(_Float16)1.f, (_Float16)1.f}, l,
                                   false);
  l = sum32(l);
  f16x o[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) {
#pragma unroll
    for (int r = 0; r < 16; ++r) o[t][r] = 0.f;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const h8 a0 = (h8){vf[t][hf][0][0], vf[t][hf][0][1], vf[t][hf][0][2], vf[t][hf][0][3],
                         vf[t][hf][1][0], vf[t][hf][1][1], vf[t][hf][1][2], vf[t][hf][1][3]};
      const h8 a1 = (h8){vf[t][hf][2][0], vf[t][hf][2][1], vf[t][hf][2][2], vf[t][hf][2][3],
                         vf[t][hf][3][0], vf[t][hf][3][1], vf[t][hf][3][2], vf[t][hf][3][3]};
      o[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, pb[hf][0], o[t], 0, 0, 0);
      o[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, pb[hf][1], o[t], 0, 0, 0);
    }
  }
  if (l32 >= G) return;
  // lane: head l32, dims t*32 + 8 rq + 4 hi + 0..3
  if (DIRECT) {
    const float inv = 1.0f / l;
    const size_t ob = (size_t)m * p.ldo + (size_t)(g * G + l32) * HD;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d0 = t * 32 + 8 * rq + 4 * hi;
        if (d0 < HD) {
          const f4 v = {o[t][4 * rq] * inv, o[t][4 * rq + 1] * inv, o[t][4 * rq + 2] * inv, o[t][4 * rq + 3] * inv};
          if (p.o32) *(f4 *)(p.o32 + ob + d0) = v;
          if (p.o16) *(h4 *)(p.o16 + ob + d0) = (h4){(_Float16)v.x, (_Float16)v.y, (_Float16)v.z, (_Float16)v.w};
        }
      }
  } else {
    constexpr int rec = attn_rec_floats(G, HD);
    float *part = p.part.buf + (((size_t)m * p.d.nkv + g) * p.part.n_chunks + c) * rec;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d0 = t * 32 + 8 * rq + 4 * hi;
        if (d0 < HD)
          *(f4 *)(part + l32 * HD + d0) = (f4){o[t][4 * rq], o[t][4 * rq + 1], o[t][4 * rq + 2], o[t][4 * rq + 3]};
      }
    if (hi == 0) {
      part[G * HD + l32] = mx * 0.6931471805599453f;  // (natural-log units, as the merges expect)
      part[G * HD + G + l32] = l;
    }
  }
}

// Combines the splits of each (row, query head): O = sum_c e^(m_c - M) o_c /
// sum_c e^(m_c - M) l_c with M the largest split maximum.  One block per
// (query head, row): the chunk weights are computed in parallel (one chunk
// per thread) and kept in LDS, then each output dimension is summed over the
// chunks by HD-thread groups that split the chunk range, and the groups'
// sums are added through LDS.  (A thread per output walking every chunk in
// turn took 60 us per layer at 4096 positions.)  k_merge_wo merges the same
// way.
template <int HD>
__global__ __launch_bounds__(256) void k_attn_merge(AttnDecP p) {
  constexpr int PARTS = 256 / HD;  // thread groups splitting the chunks
  __shared__ float sW[kMaxMergeChunks];
  __shared__ float sRed[256];
  __shared__ float sAcc[PARTS][HD];
  const int head = blockIdx.x, m = blockIdx.y;
  const int G = p.d.group, g = head / G, hg = head - g * G;
  const int tid = threadIdx.x;
  const int P = p.rows.pos[m] + 1;
  const int nch = (P + kChunkKeys - 1) / kChunkKeys;
  const int rec = attn_rec_floats(G, HD);
  const float *base = p.part.buf + ((size_t)m * p.d.nkv + g) * p.part.n_chunks * rec;
  const int om = G * HD, ol = G * HD + G;  // offsets of the maxima and the exp-sums
  const int lane = tid & 63, w = tid >> 6;

  // The first CB chunks of each thread group's share are loaded together
  // with the maxima and exp-sums, all at clamped chunks (a load tied to a
  // condition is waited for on the spot): one memory round trip for up to
  // PARTS CB chunks; longer rows read the rest after.
  constexpr int CB = HD >= 64 ? 32 : 8;
  const int dd = tid % HD, part = tid / HD;
  const float *ob = base + (size_t)hg * HD + dd;
  const float mc = base[(size_t)min(tid, nch - 1) * rec + om + hg];
  const float lc = base[(size_t)min(tid, nch - 1) * rec + ol + hg];
  float ov[CB];
#pragma unroll
  for (int i = 0; i < CB; ++i) ov[i] = ob[(size_t)min(part + PARTS * i, nch - 1) * rec];
  float mx = kNegInf;
  for (int c = tid; c < nch; c += 256) mx = fmaxf(mx, c == tid ? mc : base[(size_t)c * rec + om + hg]);
  mx = wave_max(mx);
  if (lane == 0) sRed[w] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(sRed[0], sRed[1]), fmaxf(sRed[2], sRed[3]));
  float l = 0.f;
  for (int c = tid; c < nch; c += 256) {
    const float *r = base + (size_t)c * rec;
    const float wgt = __expf((c == tid ? mc : r[om + hg]) - M);
    sW[c] = wgt;
    l = fmaf(c == tid ? lc : r[ol + hg], wgt, l);
  }
  l = wave_sum(l);
  if (lane == 0) sRed[4 + w] = l;
  __syncthreads();
  const float L = (sRed[4] + sRed[5]) + (sRed[6] + sRed[7]);

  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < CB; ++i)
    if (part + PARTS * i < nch) acc = fmaf(ov[i], sW[part + PARTS * i], acc);
#pragma unroll 4
  for (int c = part + PARTS * CB; c < nch; c += PARTS) acc = fmaf(ob[(size_t)c * rec], sW[c], acc);
  sAcc[part][dd] = acc;
  __syncthreads();
  if (tid < HD) {
    float v = 0.f;
#pragma unroll
    for (int q = 0; q < PARTS; ++q) v += sAcc[q][tid];
    v /= L;
    const size_t oi = (size_t)m * p.ldo + (size_t)head * HD + tid;
    if (p.o32) p.o32[oi] = v;
    if (p.o16) p.o16[oi] = (_Float16)v;
  }
}

// ------------------------------------------------- attention fused with WO
// For short contexts (all rows at positions < kFusedKeys) on the decode
// path: one block per (WO row chunk, query head).  The block computes its
// head's attention output for every row (online softmax over 256-key tiles:
// thread t scores key t, wavefront w and lane d accumulate P.V for keys
// 64w..64w+63 of the tile), then multiplies it by its slice of WO,
// WO[chunk rows, head columns], and adds the partial sums into the residual
// rows with float atomics.  Nothing reads the residual while this kernel
// runs, so the adds only race with each other (summation order varies by an
// ulp from run to run).  The WO slice is loaded at kernel start, so its
// latency overlaps the attention.
struct AttnWoP {
  Dims d;
  int layer;
  KVCache kv;
  const float *q;
  int ldq;
  RowInfo rows;
  int M;
  const _Float16 *wo;
  float *h;
  int ldh;
  int rows_per_block;
  float scale;
  // One-row calls (k_attn_wo1): K and V of KV head 0 of the row's (layer,
  // sequence) block (head g starts g * n_ctx * HD floats later) and the
  // number of key slots nk1 its loads cover (the row's position < nk1 <=
  // n_ctx), known on the host; the position itself is read on the device.
  const float *kb1, *vb1;
  int nk1;
  L2Warm warm;   // one-row calls: producer blocks in grid rows y >= nh (the down projection)
  L2Warm warm2;  // ... and after them (the next layer's QKV projection)
};

template <int N>
__device__ __forceinline__ float group_sum(float v) {  // sum within aligned groups of N lanes
  if (N >= 2) v += dpp<0xB1>(v);
  if (N >= 4) v += dpp<0x4E>(v);
  if (N >= 8) v += dpp<0x141>(v);
  if (N >= 16) v += dpp<0x140>(v);
  return v;
}

template <int HD, int MT>
__global__ __launch_bounds__(256) void k_attn_wo(AttnWoP p) {
  constexpr int TK = HD >= 128 ? 128 : 256;  // keys per tile (one per thread up to TK)
  constexpr int C4 = HD / 4;                 // 16-byte chunks per K row
  constexpr int KPT = TK * C4 / 256;         // K chunks loaded per thread
  constexpr int KW = TK / 4;                 // keys per wavefront in P.V
  // P.V: a lane holds 4 consecutive dims (one 16-byte load per key), LD lanes
  // cover a V row and the PH lane groups of a wavefront take interleaved keys,
  // so a lane issues KPL 16-byte V loads (K: KPT, WO: 8; all within the 63
  // loads a wavefront can have outstanding).
  constexpr int LD = HD / 4;
  constexpr int PH = 64 / LD;
  constexpr int KPL = KW / PH;
  constexpr int LPR = HD / 8;              // lanes per WO row segment (8 halves each)
  constexpr int RPI = 64 / LPR;            // WO rows per wavefront load
  constexpr int WI = wo_loads_fused(HD);  // WO loads per wavefront
  // K tile in LDS, 16-byte chunk c of key row j stored at chunk c ^ (j % C4):
  // a lane walking its own row meets a different bank group than its
  // neighbours, so the row reads are conflict-free without padding.
  __shared__ f4 sK[TK * C4];
  __shared__ __attribute__((aligned(16))) float sQ[HD];
  __shared__ float sP[TK];
  __shared__ float sRed[2][4];
  __shared__ __attribute__((aligned(16))) float sOp[4 * PH * HD];
  __shared__ __attribute__((aligned(16))) float sO[MT * HD];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int rc = blockIdx.x, head = blockIdx.y;
  const int G = p.d.group, H = p.d.H, nhd = p.d.nh * HD;
  const int g = head / G;
  const int M = p.M;
  // Every kernel argument the loads below need, requested in the first
  // scalar-load batch (the empty asm uses them here, so none of them is left
  // to a later batch, whose round trip would come before the loads).
  {
    const int *rp = p.rows.pos, *rs = p.rows.seq;
    const float *qp = p.q, *kp = p.kv.k, *vp = p.kv.v;
    const _Float16 *wp = p.wo;
    asm volatile("" ::"s"(rp), "s"(rs), "s"(qp), "s"(kp), "s"(vp), "s"(wp));
    asm volatile("" ::"s"(G), "s"(H), "s"(p.d.nh), "s"(p.d.nkv), "s"(p.d.n_seq), "s"(p.d.n_ctx),
                 "s"(p.layer), "s"(p.rows_per_block), "s"(p.scale));
  }

  // WO slice loads first
  const int r0 = rc * p.rows_per_block;
  const int rend = min(H, r0 + p.rows_per_block);
  const int kc = lane % LPR;
  // Loads are unconditional, at clamped indices, with no select on their
  // values (a load the compiler can tie to a condition is moved into a
  // branch, and its value is then copied at the branch join, which waits for
  // it on the spot): WO rows past the chunk are never stored, keys past the
  // position re-read the last visible key (a cache hit) and get a -inf
  // score and a zero weight.  The first row's position,
  // sequence slot and q go out before the WO slice, so the K / V loads that
  // depend on them do not wait for the slice (vector loads complete in order).
  const int d_lane = lane % LD, ph = lane / LD;
  int pos = (int)vload(p.rows.pos, 0), seq = (int)vload(p.rows.seq, 0);
  float qraw = p.q[(size_t)head * HD + (tid < HD ? tid : 0)];
  __builtin_amdgcn_sched_barrier(0);  // (keeps this issue order)
  h8 wreg[WI];
#pragma unroll
  for (int i = 0; i < WI; ++i) {
    const int row = r0 + (w * WI + i) * RPI + lane / LPR;
    wreg[i] = __builtin_nontemporal_load(
        (const h8 *)(p.wo + (size_t)min(row, H - 1) * nhd + (size_t)head * HD + kc * 8));
  }

  const int M_rows = MT == 1 ? 1 : M;  // (one row: no reload path in the loop)
  for (int m = 0; m < M_rows; ++m) {
    if (m > 0) {
      pos = (int)vload(p.rows.pos, m);
      seq = (int)vload(p.rows.seq, m);
      qraw = p.q[(size_t)m * p.ldq + (size_t)head * HD + (tid < HD ? tid : 0)];
    }
    const int P = pos + 1;
    const f4 *kbase = (const f4 *)(p.kv.k + p.kv.off(p.d, p.layer, seq, g, 0));
    const float *vbase = p.kv.v + p.kv.off(p.d, p.layer, seq, g, 0);
    float m_run = kNegInf, l_run = 0.f;
    f4 o = {0.f, 0.f, 0.f, 0.f};
    int t0 = 0;
    do {
      // this tile's K chunks (coalesced) and the V values of this lane's keys
      f4 kr[KPT];
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const int ci = tid + 256 * i, j = ci / C4;
        kr[i] = kbase[(size_t)min(t0 + j, P - 1) * C4 + (ci - j * C4)];
      }
      f4 v[KPL];
#pragma unroll
      for (int i = 0; i < KPL; ++i) {
        const int jj = t0 + KW * w + ph + PH * i;
        v[i] = *(const f4 *)(vbase + (size_t)min(jj, P - 1) * HD + 4 * d_lane);
      }
      const float qv = tid < HD ? qraw * p.scale : 0.f;
      __syncthreads();  // the previous tile's (or row's) LDS reads are done
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const int ci = tid + 256 * i, j = ci / C4, c = ci - j * C4;
        sK[j * C4 + (c ^ (j % C4))] = kr[i];
      }
      if (tid < HD) sQ[tid] = qv;
      __syncthreads();
      const int j = t0 + tid;
      float s = kNegInf;
      if (tid < TK && j < P) {
        float a = 0.f;
#pragma unroll
        for (int c = 0; c < C4; ++c) {
          const f4 kv4 = sK[tid * C4 + (c ^ (tid % C4))];
          const f4 q4 = *(const f4 *)(sQ + 4 * c);
          a = fmaf(q4.x, kv4.x, fmaf(q4.y, kv4.y, fmaf(q4.z, kv4.z, fmaf(q4.w, kv4.w, a))));
        }
        s = a;
      }
      const float wm = wave_max(s);
      if (lane == 0) sRed[0][w] = wm;
      __syncthreads();
      const float mx = fmaxf(fmaxf(sRed[0][0], sRed[0][1]), fmaxf(sRed[0][2], sRed[0][3]));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __expf(m_run - m_new);
      const float e = (tid < TK && j < P) ? __expf(s - m_new) : 0.f;
      if (tid < TK) sP[tid] = e;
      const float ws = wave_sum(e);
      if (lane == 0) sRed[1][w] = ws;
      __syncthreads();
      const float sum = (sRed[1][0] + sRed[1][1]) + (sRed[1][2] + sRed[1][3]);
      l_run = l_run * alpha + sum;
      m_run = m_new;
      o *= alpha;
#pragma unroll
      for (int i = 0; i < KPL; ++i) o += sP[KW * w + ph + PH * i] * v[i];
      t0 += TK;
    } while (t0 < P);
    __syncthreads();  // sOp of the previous row is consumed
    *(f4 *)(sOp + (w * PH + ph) * HD + 4 * d_lane) = o;
    __syncthreads();
    if (tid < HD) {
      float acc = 0.f;
#pragma unroll
      for (int k = 0; k < 4 * PH; ++k) acc += sOp[k * HD + tid];
      sO[m * HD + tid] = acc / l_run;
    }
  }
  __syncthreads();

  // WO slice times the head outputs; partial row sums added into the residual
#pragma unroll
  for (int i = 0; i < WI; ++i) {
    const int row = r0 + (w * WI + i) * RPI + lane / LPR;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m < M) {
        const f4 o0 = *(const f4 *)(sO + m * HD + kc * 8);
        const f4 o1 = *(const f4 *)(sO + m * HD + kc * 8 + 4);
        float a = (float)wreg[i][0] * o0.x;
        a = fmaf((float)wreg[i][1], o0.y, a);
        a = fmaf((float)wreg[i][2], o0.z, a);
        a = fmaf((float)wreg[i][3], o0.w, a);
        a = fmaf((float)wreg[i][4], o1.x, a);
        a = fmaf((float)wreg[i][5], o1.y, a);
        a = fmaf((float)wreg[i][6], o1.z, a);
        a = fmaf((float)wreg[i][7], o1.w, a);
        a = group_sum<LPR>(a);
        if (kc == 0 && row < rend) atomicAdd(p.h + (size_t)m * p.ldh + row, a);
      }
    }
  }
}

// Sum of v over the lanes l with the same l % N (N a power of two, 4..32):
// the other lanes of the wavefront hold other keys' partial sums for the
// same dimensions.
template <int N>
__device__ __forceinline__ float across_groups(float v) {
  if (N < 16) {  // (only head_dim 16: 4 lanes per key)
    for (int o = N; o < 16; o <<= 1) v += __shfl_xor(v, o, 64);
  }
  if (N < 32) {
    float a, b;
    pair16(v, a, b);
    v = a + b;
  }
  return sum32(v);
}

// One row (batch-1 decode, a prefill's last row): one block per (WO row
// chunk, query head), as k_attn_wo, with a shorter critical path.  The
// host gives the row's K / V block and a key bound nk1, so every load of
// the block (q, the WO slice, the position and the K / V of its first key
// tile) is issued at once, before any of them is waited for.  A key's
// score is computed where its K row lands: HD / 4 lanes hold 4 dimensions
// each and combine their partial dot products with DPP, so K never goes
// through LDS; softmax and P.V stay in registers, and the four wavefronts
// meet twice per call (the tile maximum, then the outputs).  Keys past the
// position get a -inf score and a zero V (a select, so whatever a slot past
// the position holds cannot reach the sums).
template <int HD>
__global__ __launch_bounds__(256) void k_attn_wo1(AttnWoP p) {
  constexpr int LPK = HD / 4;             // lanes per key (4 dims, one 16-byte load, each)
  constexpr int KPI = 64 / LPK;           // keys per wavefront load
  constexpr int NI = HD == 16 ? 8 : 16;   // K (and V) loads per lane and key tile
  constexpr int KPW = NI * KPI;           // keys per wavefront and tile
  constexpr int TK = 4 * KPW;             // keys per tile: 256 (hd 64), 128 (hd 128), 512 (hd 16)
  constexpr int LPR = HD / 8;             // lanes per WO row segment (8 halves each)
  constexpr int RPI = 64 / LPR;           // WO rows per wavefront load
  constexpr int WI = wo_loads_fused(HD);  // WO loads per wavefront
  __shared__ float sM[2][4];
  __shared__ float sL[4];
  __shared__ __attribute__((aligned(16))) float sO[4][HD];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int rc = blockIdx.x, head = blockIdx.y;
  const int G = p.d.group, H = p.d.H, nhd = p.d.nh * HD;
  const int g = head / G;
  const int dc = lane % LPK, kg = lane / LPK;
  {  // the kernel arguments the loads need, in the first scalar-load batch
    const int *rp = p.rows.pos;
    const float *qp = p.q, *kp = p.kb1, *vp = p.vb1;
    const _Float16 *wp = p.wo;
    asm volatile("" ::"s"(rp), "s"(qp), "s"(kp), "s"(vp), "s"(wp));
    asm volatile("" ::"s"(G), "s"(H), "s"(p.d.nh), "s"(p.d.n_ctx), "s"(p.nk1),
                 "s"(p.rows_per_block), "s"(p.scale));
  }
  if (head >= p.d.nh) {  // an L2 warming producer (grid rows past the heads)
    const int id = rc + head * (int)gridDim.x;
    if (id < p.warm.p0 + p.warm.n_prod)
      l2_warm<kWarmStepsAttn>(p.warm, id);
    else
      l2_warm<kWarmStepsAttn>(p.warm2, id);
    return;
  }
  const unsigned pos = vload(p.rows.pos, 0);
  const f4 q4 = *(const f4 *)(p.q + (size_t)head * HD + 4 * dc);
  const int r0 = rc * p.rows_per_block;
  const int rend = min(H, r0 + p.rows_per_block);
  const int kc = lane % LPR;
  h8 wreg[WI];
#pragma unroll
  for (int i = 0; i < WI; ++i) {
    const int row = r0 + (w * WI + i) * RPI + lane / LPR;
    wreg[i] = __builtin_nontemporal_load(
        (const h8 *)(p.wo + (size_t)min(row, H - 1) * nhd + (size_t)head * HD + kc * 8));
  }
  const float *kb = p.kb1 + (size_t)g * p.d.n_ctx * HD + 4 * dc;
  const float *vb = p.vb1 + (size_t)g * p.d.n_ctx * HD + 4 * dc;
  const int klast = p.nk1 - 1;

  float m_run = kNegInf, l_run = 0.f;
  f4 o = {0.f, 0.f, 0.f, 0.f};
  int t0 = 0, tile = 0;
  unsigned pos_t;
  do {
    f4 kr[NI], vr[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int key = min(t0 + w * KPW + i * KPI + kg, klast);
      kr[i] = *(const f4 *)(kb + (size_t)key * HD);
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int key = min(t0 + w * KPW + i * KPI + kg, klast);
      vr[i] = *(const f4 *)(vb + (size_t)key * HD);
    }
    __builtin_amdgcn_sched_barrier(0);  // (every load of the tile issued before any use)
    // The position, passed through an empty asm here: otherwise the
    // compiler derives the trip count from it before the loop, which waits
    // for its load ahead of the K / V loads.
    pos_t = pos;
    asm volatile("" : "+v"(pos_t));
    // scores of this lane group's NI keys (each in all LPK lanes of the group)
    float sc[NI];
    float mt = kNegInf;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float a = q4.x * kr[i].x;
      a = fmaf(q4.y, kr[i].y, a);
      a = fmaf(q4.z, kr[i].z, a);
      a = fmaf(q4.w, kr[i].w, a);
      a = group_sum<LPK < 16 ? LPK : 16>(a);
      if (LPK == 32) {  // (a key's 32 lanes: rows l and l ^ 16 of a half)
        float x, y;
        pair16(a, x, y);
        a = x + y;
      }
      const unsigned key = (unsigned)(t0 + w * KPW + i * KPI + kg);
      sc[i] = key <= pos_t ? a * p.scale : kNegInf;
      mt = fmaxf(mt, sc[i]);
    }
    mt = wave_max(mt);
    if (lane == 0) sM[tile & 1][w] = mt;
    __syncthreads();
    const float mx = fmaxf(fmaxf(sM[tile & 1][0], sM[tile & 1][1]),
                           fmaxf(sM[tile & 1][2], sM[tile & 1][3]));
    const float m_new = fmaxf(m_run, mx);  // (finite: key t0 <= pos is in every tile)
    const float alpha = __expf(m_run - m_new);
    float lt = 0.f;
    f4 ot = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const float e = __expf(sc[i] - m_new);
      const unsigned key = (unsigned)(t0 + w * KPW + i * KPI + kg);
      const f4 vv = key <= pos_t ? vr[i] : (f4){0.f, 0.f, 0.f, 0.f};
      lt += e;
      ot += e * vv;
    }
    l_run = l_run * alpha + lt;
    o = o * alpha + ot;
    m_run = m_new;
    t0 += TK;
    ++tile;
  } while ((unsigned)t0 <= pos_t);

  // this wavefront's sums over all its keys, then over the four wavefronts
  o.x = across_groups<LPK>(o.x);
  o.y = across_groups<LPK>(o.y);
  o.z = across_groups<LPK>(o.z);
  o.w = across_groups<LPK>(o.w);
  l_run = across_groups<LPK>(l_run);
  if (kg == 0) *(f4 *)&sO[w][4 * dc] = o;
  if (lane == 0) sL[w] = l_run;
  __syncthreads();
  const float inv = 1.0f / ((sL[0] + sL[1]) + (sL[2] + sL[3]));
  f4 o0 = *(const f4 *)&sO[0][kc * 8], o1 = *(const f4 *)&sO[0][kc * 8 + 4];
#pragma unroll
  for (int ww = 1; ww < 4; ++ww) {
    o0 += *(const f4 *)&sO[ww][kc * 8];
    o1 += *(const f4 *)&sO[ww][kc * 8 + 4];
  }
  o0 *= inv;
  o1 *= inv;

  // WO slice times the head output; partial row sums added into the residual
#pragma unroll
  for (int i = 0; i < WI; ++i) {
    const int row = r0 + (w * WI + i) * RPI + lane / LPR;
    float a = (float)wreg[i][0] * o0.x;
    a = fmaf((float)wreg[i][1], o0.y, a);
    a = fmaf((float)wreg[i][2], o0.z, a);
    a = fmaf((float)wreg[i][3], o0.w, a);
    a = fmaf((float)wreg[i][4], o1.x, a);
    a = fmaf((float)wreg[i][5], o1.y, a);
    a = fmaf((float)wreg[i][6], o1.z, a);
    a = fmaf((float)wreg[i][7], o1.w, a);
    a = group_sum<LPR>(a);
    if (kc == 0 && row < rend) atomicAdd(p.h + row, a);
  }
}

template <int HD>
static void attn_wo_hd(const AttnWoP &p, int grid_x, hipStream_t st) {
  dim3 grid(grid_x, p.d.nh);
  if (p.M <= 1) {
    grid.y += (p.warm.n_prod + p.warm2.n_prod) / grid_x;  // (n_prod: whole grid rows)
    hipLaunchKernelGGL((k_attn_wo1<HD>), grid, dim3(256), 0, st, p);
  } else {
    hipLaunchKernelGGL((k_attn_wo<HD, 8>), grid, dim3(256), 0, st, p);
  }
}

void attn_wo_fused(const Dims &d, int layer, const KVCache &kv, const float *q, int ldq,
                   RowInfo rows, int M, int seq1, int nk1, const uint16_t *wo, float *h, int ldh,
                   const uint16_t *warm_wd, const uint16_t *warm_wqkv, hipStream_t st) {
  const int rpb = 4 * wo_loads_fused(d.hd) * (64 / (d.hd / 8));  // WO rows per block
  AttnWoP p{d, layer, kv, q, ldq, rows, M, (const _Float16 *)wo, h, ldh, rpb,
            1.0f / sqrtf((float)d.hd), nullptr, nullptr, 0, L2Warm{}, L2Warm{}};
  const int gx = (d.H + rpb - 1) / rpb;
  if (M <= 1) {
    p.kb1 = kv.k + kv.off(d, layer, seq1, 0, 0);
    p.vb1 = kv.v + kv.off(d, layer, seq1, 0, 0);
    p.nk1 = nk1;
    if (warm_wd)  // whole grid rows of producers after the heads' rows
      p.warm = warm_gemv1(warm_wd, d.H, d.I_pad, down_rows1(d.I_pad), gx * d.nh,
                          kWarmProdAttn / gx * gx, kWarmStepsAttn);
    if (warm_wqkv)  // then the next layer's QKV rows (its one-row GEMV: 2 rows per wave)
      p.warm2 = warm_gemv1(warm_wqkv, d.nqkv, d.H, 2, gx * d.nh + p.warm.n_prod,
                           kWarmProdQkv / gx * gx, kWarmStepsAttn);
  }
  switch (d.hd) {
    case 16: attn_wo_hd<16>(p, gx, st); break;
    case 64: attn_wo_hd<64>(p, gx, st); break;
    default: attn_wo_hd<128>(p, gx, st); break;
  }
}

// ------------------------------------- chunk-record merge fused with WO
// Longer contexts on the decode path: after k_attn_decode_mfma has left its
// chunk records, one block per (WO row chunk, query head) merges the head's
// records into its attention output (as k_attn_merge does) and multiplies it
// by its slice of WO, adding the partial row sums into the residual with
// float atomics (as k_attn_wo).  This replaces the merge kernel and the WO
// GEMV, one kernel boundary fewer per layer.  The WO slice is loaded first,
// so its latency overlaps the merge.
struct MergeWoP {
  Dims d;
  AttnPartials part;
  RowInfo rows;
  int M;
  const _Float16 *wo;
  float *h;
  int ldh;
  int rows_per_block;
};

template <int HD, int MT>
__global__ __launch_bounds__(256) void k_merge_wo(MergeWoP p) {
  constexpr int PARTS = 256 / HD;          // thread groups splitting the chunks
  constexpr int LPR = HD / 8;              // lanes per WO row segment (8 halves each)
  constexpr int RPI = 64 / LPR;            // WO rows per wavefront load
  constexpr int WI = wo_loads_per_wave(HD);  // WO loads per wavefront
  __shared__ float sW[kMaxMergeChunks];
  __shared__ float sRed[2][4];
  __shared__ float sAcc[PARTS][HD];
  __shared__ __attribute__((aligned(16))) float sO[MT * HD];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int rc = blockIdx.x, head = blockIdx.y;
  const int G = p.d.group, g = head / G, hg = head - g * G;
  const int H = p.d.H, nhd = p.d.nh * HD;

  const int r0 = rc * p.rows_per_block;
  const int rend = min(H, r0 + p.rows_per_block);
  const int kc = lane % LPR;
  h8 wreg[WI];
#pragma unroll
  for (int i = 0; i < WI; ++i) {
    const int row = r0 + (w * WI + i) * RPI + lane / LPR;
    wreg[i] = __builtin_nontemporal_load(
        (const h8 *)(p.wo + (size_t)min(row, H - 1) * nhd + (size_t)head * HD + kc * 8));
  }

  const int rec = attn_rec_floats(G, HD);
  const int om = G * HD, ol = G * HD + G;  // offsets of the maxima and the exp-sums
  // The first CB chunks of each thread group's share are loaded together
  // with the maxima and exp-sums (one memory round trip for up to PARTS CB
  // chunks: 64 at hd 128, 128 at hd 64); longer rows read the rest after.
  constexpr int CB = HD >= 64 ? 32 : 8;
  const int dd = tid % HD, part = tid / HD;
  const int M_rows = MT == 1 ? 1 : p.M;
  for (int m = 0; m < M_rows; ++m) {
    const int P = p.rows.pos[m] + 1;
    const int nch = (P + kChunkKeys - 1) / kChunkKeys;
    const float *base = p.part.buf + ((size_t)m * p.d.nkv + g) * p.part.n_chunks * rec;
    const float *ob = base + (size_t)hg * HD + dd;
    // (unconditional loads at clamped chunks: a load tied to a condition is
    // waited for on the spot; only chunks < nch are used)
    float mx = kNegInf;
    const float mc = base[(size_t)min(tid, nch - 1) * rec + om + hg];
    const float lc = base[(size_t)min(tid, nch - 1) * rec + ol + hg];
    float ov[CB];
#pragma unroll
    for (int i = 0; i < CB; ++i) ov[i] = ob[(size_t)min(part + PARTS * i, nch - 1) * rec];
    for (int c = tid; c < nch; c += 256) mx = fmaxf(mx, c == tid ? mc : base[(size_t)c * rec + om + hg]);
    mx = wave_max(mx);
    __syncthreads();  // (the previous row's reads of sW, sAcc and sRed are done)
    if (lane == 0) sRed[0][w] = mx;
    __syncthreads();
    const float Mx = fmaxf(fmaxf(sRed[0][0], sRed[0][1]), fmaxf(sRed[0][2], sRed[0][3]));
    float l = 0.f;
    for (int c = tid; c < nch; c += 256) {
      const float *r = base + (size_t)c * rec;
      const float wgt = __expf((c == tid ? mc : r[om + hg]) - Mx);
      sW[c] = wgt;
      l = fmaf(c == tid ? lc : r[ol + hg], wgt, l);
    }
    l = wave_sum(l);
    if (lane == 0) sRed[1][w] = l;
    __syncthreads();
    const float L = (sRed[1][0] + sRed[1][1]) + (sRed[1][2] + sRed[1][3]);
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < CB; ++i)
      if (part + PARTS * i < nch) acc = fmaf(ov[i], sW[part + PARTS * i], acc);
#pragma unroll 4
    for (int c = part + PARTS * CB; c < nch; c += PARTS) acc = fmaf(ob[(size_t)c * rec], sW[c], acc);
    sAcc[part][dd] = acc;
    __syncthreads();
    if (tid < HD) {
      float v = 0.f;
#pragma unroll
      for (int q = 0; q < PARTS; ++q) v += sAcc[q][tid];
      sO[m * HD + tid] = v / L;
    }
  }
  __syncthreads();

  // WO slice times the head outputs; partial row sums added into the residual
#pragma unroll
  for (int i = 0; i < WI; ++i) {
    const int row = r0 + (w * WI + i) * RPI + lane / LPR;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m < p.M) {
        const f4 o0 = *(const f4 *)(sO + m * HD + kc * 8);
        const f4 o1 = *(const f4 *)(sO + m * HD + kc * 8 + 4);
        float a = (float)wreg[i][0] * o0.x;
        a = fmaf((float)wreg[i][1], o0.y, a);
        a = fmaf((float)wreg[i][2], o0.z, a);
        a = fmaf((float)wreg[i][3], o0.w, a);
        a = fmaf((float)wreg[i][4], o1.x, a);
        a = fmaf((float)wreg[i][5], o1.y, a);
        a = fmaf((float)wreg[i][6], o1.z, a);
        a = fmaf((float)wreg[i][7], o1.w, a);
        a = group_sum<LPR>(a);
        if (kc == 0 && row < rend) atomicAdd(p.h + (size_t)m * p.ldh + row, a);
      }
    }
  }
}

template <int HD>
static void merge_wo_hd(const MergeWoP &p, int grid_x, hipStream_t st) {
  dim3 grid(grid_x, p.d.nh);
  if (p.M <= 1)
    hipLaunchKernelGGL((k_merge_wo<HD, 1>), grid, dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL((k_merge_wo<HD, 8>), grid, dim3(256), 0, st, p);
}

void merge_wo(const Dims &d, const AttnPartials &part, RowInfo rows, int M, const uint16_t *wo,
              float *h, int ldh, hipStream_t st) {
  const int rpb = 4 * wo_loads_per_wave(d.hd) * (64 / (d.hd / 8));  // WO rows per block
  const MergeWoP p{d, part, rows, M, (const _Float16 *)wo, h, ldh, rpb};
  const int gx = (d.H + rpb - 1) / rpb;
  switch (d.hd) {
    case 16: merge_wo_hd<16>(p, gx, st); break;
    case 64: merge_wo_hd<64>(p, gx, st); break;
    default: merge_wo_hd<128>(p, gx, st); break;
  }
}

template <int HD, int G>
static void attn_decode_g(const AttnDecP &p, int M, int n_chunks, bool merge, hipStream_t st) {
  if (n_chunks <= 1) {
    hipLaunchKernelGGL((k_attn_decode_mfma<HD, G, true>), dim3(1, p.d.nkv, M), dim3(64), 0, st, p);
  } else {
    hipLaunchKernelGGL((k_attn_decode_mfma<HD, G, false>), dim3(n_chunks, p.d.nkv, M), dim3(64), 0,
                       st, p);
    if (merge) hipLaunchKernelGGL((k_attn_merge<HD>), dim3(p.d.nh, M), dim3(256), 0, st, p);
  }
}

template <int HD>
static void attn_decode_hd(const AttnDecP &p, int M, int n_chunks, bool merge, hipStream_t st) {
  switch (p.d.group) {  // the group size is a compile-time constant of the kernel
    case 1: attn_decode_g<HD, 1>(p, M, n_chunks, merge, st); break;
    case 2: attn_decode_g<HD, 2>(p, M, n_chunks, merge, st); break;
    case 3: attn_decode_g<HD, 3>(p, M, n_chunks, merge, st); break;
    case 4: attn_decode_g<HD, 4>(p, M, n_chunks, merge, st); break;
    case 5: attn_decode_g<HD, 5>(p, M, n_chunks, merge, st); break;
    case 6: attn_decode_g<HD, 6>(p, M, n_chunks, merge, st); break;
    case 7: attn_decode_g<HD, 7>(p, M, n_chunks, merge, st); break;
    default: attn_decode_g<HD, 8>(p, M, n_chunks, merge, st); break;
  }
}

void attn_decode(const Dims &d, int layer, const KVCache &kv, const float *q, int ldq,
                 RowInfo rows, int M, int n_chunks, bool merge, const AttnPartials &part,
                 float *o32, _Float16 *o16, int ldo, hipStream_t st) {
  AttnDecP p{d, layer, kv, q, ldq, rows, part, o32, o16, ldo, 1.0f / sqrtf((float)d.hd)};
  switch (d.hd) {
    case 16: attn_decode_hd<16>(p, M, n_chunks, merge, st); break;
    case 64: attn_decode_hd<64>(p, M, n_chunks, merge, st); break;
    default: attn_decode_hd<128>(p, M, n_chunks, merge, st); break;
  }
}

// ------------------------------------------------------------------ prefill
// Causal flash attention on v_mfma_f32_32x32x16_f16 for one prefill pass of
// one sequence, on the binary16 mirror of the cache (K as [pos][d], V
// transposed as [d][pos]: the MFMA operand layouts; written by every K/V
// store, and by k_kv_f16 after a direct write of the f32 cache).  One block
// per (32-query tile, KV head) with one wavefront per query head of the
// group (G = group size), so each K / V tile in LDS serves the whole group;
// short prompts (fewer than 128 such blocks) instead run one block per query
// head (G = 1, blockIdx.z = head within the group), trading repeated K / V
// tile loads for seven times the blocks.  Per 64-key tile and 32-key half:
//   S^T[key, query] = K (A: 32 keys x 16 d) * Q^T (B: 16 d x 32 queries)
// so each lane owns one query column and 16 of the half's keys (the other 16
// sit in lane ^ 32): the online-softmax max and sum need one cross-lane step,
// and the probabilities are already in the B-operand layout of
//   O^T[d, query] += V^T (A: 32 d x 16 keys) * P^T (B: 16 keys x 32 queries)
// once V^T's key order is matched to the lanes' key order.  Key tiles are
// double-buffered in LDS (loads of tile t+2 in flight while tile t is
// multiplied; one barrier per tile).  Accumulation stays in f32.
// MFMA 32x32 operand layout: lane l supplies A[l%32][8*(l/32)..+8] and
// B[8*(l/32)..+8][l%32]; it receives D[8*(r/4) + 4*(l/32) + r%4][l%32], r<16.
constexpr int kPreKeys = 64;  // keys per tile of the prefill attention

struct KvF16P {
  Dims d;
  int layer, seq, pos0, n;
  KVCache kv;
};

// One block per (64 positions, KV head) of the range: K rows are converted
// in place order, V through an LDS transpose.
template <int HD>
__global__ __launch_bounds__(256) void k_kv_f16(KvF16P p) {
  __shared__ float sT[HD][kPreKeys + 1];
  const int g = blockIdx.y, p0 = p.pos0 + blockIdx.x * kPreKeys;
  const int np = min(kPreKeys, p.pos0 + p.n - p0);
  const int tid = threadIdx.x;
  const float *kb = p.kv.k + p.kv.off(p.d, p.layer, p.seq, g, 0);
  const float *vb = p.kv.v + p.kv.off(p.d, p.layer, p.seq, g, 0);
  const size_t b16 = p.kv.off16(p.d, p.layer, p.seq, g);
  _Float16 *ko = p.kv.k16 + b16 + (size_t)p0 * HD;
  for (int i = tid; i < np * HD; i += 256) {
    const int pp = i / HD, dd = i - pp * HD;
    ko[i] = (_Float16)kb[(size_t)(p0 + pp) * HD + dd];
    sT[dd][pp] = vb[(size_t)(p0 + pp) * HD + dd];
  }
  __syncthreads();
  _Float16 *vo = p.kv.v16t + b16 + p0;
  for (int i = tid; i < kPreKeys * HD; i += 256) {
    const int dd = i / kPreKeys, pp = i - dd * kPreKeys;
    if (pp < np) vo[(size_t)dd * p.kv.ldp + pp] = (_Float16)sT[dd][pp];
  }
}

void kv_mirror(const Dims &d, const KVCache &kv, int layer, int seq, int pos0, int n,
               hipStream_t st) {
  const KvF16P cp{d, layer, seq, pos0, n, kv};
  const dim3 grid((n + kPreKeys - 1) / kPreKeys, d.nkv);
  switch (d.hd) {
    case 16: hipLaunchKernelGGL(k_kv_f16<16>, grid, dim3(256), 0, st, cp); break;
    case 64: hipLaunchKernelGGL(k_kv_f16<64>, grid, dim3(256), 0, st, cp); break;
    default: hipLaunchKernelGGL(k_kv_f16<128>, grid, dim3(256), 0, st, cp); break;
  }
}

// One sequence's share of a prefill-attention launch: rows r0 .. r0+M-1 of
// the pass, its (layer, sequence) block of the mirror, and its work split.
struct PreSeg {
  int r0, M;
  // causal balance: query tiles split_from .. n_tiles-1 run as two blocks
  // each (first / second half of their key tiles) whose softmax states go to
  // part (from split record part0 on) and are combined by k_attn_prefill_merge
  int n_tiles, split_from, part0;
  int p0;         // position of row r0 when the rows' positions are p0, p0+1, ...; else -1
  size_t kv_off;  // element offset of the sequence's KV head 0 in either mirror
};

// First query tile of a segment with positions p0 .. p0+M-1 (T tiles of 32
// rows) whose key-tile count (p0 + min(32 t + 31, M - 1)) / 64 + 1 is at
// least u; T if none.
__device__ __forceinline__ int tile_reaching(int p0, int M, int T, int u) {
  const int X = kPreKeys * (u - 1) - p0;  // the row the tile's last row must reach
  if (X > M - 1) return T;
  return X <= 0 ? 0 : X / 32;
}

// Work item wi of a segment with contiguous positions, taking the items in
// descending order of key tiles (longest first over whole tiles and split
// pieces together, the list-scheduling order that keeps the CUs' finishing
// times close): the item's tile and piece (-1: whole tile; 0 / 1: the
// first / second part of a split tile's key tiles, ceil / floor of half).
// Items with at least v key tiles are counted in closed form, the work
// value of item wi is found by bisection, and within one value whole tiles,
// first pieces and second pieces follow each other, each in descending
// tile order.
__device__ inline void prefill_item_lpt(const PreSeg &sg, int wi, int &tile, int &piece) {
  const int p0 = sg.p0, M = sg.M, T = sg.n_tiles, sf = sg.split_from;
  auto first = [&](int u) { return tile_reaching(p0, M, T, u); };
  auto count_ge = [&](int v) {
    return max(0, sf - first(v)) + (T - max(sf, first(2 * v - 1))) + (T - max(sf, first(2 * v)));
  };
  int lo = 1, hi = (p0 + M - 1) / kPreKeys + 2;  // count_ge(lo) > wi >= count_ge(hi)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (count_ge(mid) > wi) lo = mid;
    else hi = mid;
  }
  int r = wi - count_ge(lo + 1);  // rank among the items of exactly lo key tiles
  const int w_hi = min(first(lo + 1), sf), w_n = w_hi - min(first(lo), sf);
  if (r < w_n) {
    tile = w_hi - 1 - r;
    piece = -1;
    return;
  }
  r -= w_n;
  const int a_hi = max(sf, first(2 * lo + 1)), a_n = a_hi - max(sf, first(2 * lo - 1));
  if (r < a_n) {
    tile = a_hi - 1 - r;
    piece = 0;
    return;
  }
  r -= a_n;
  tile = max(sf, first(2 * lo + 2)) - 1 - r;
  piece = 1;
}
constexpr int kPreSegs = 8;  // sequences per launch

struct AttnPreP {
  Dims d;
  const float *q;
  int ldq;
  RowInfo rows;
  const _Float16 *k16, *v16t;  // the layer's mirrors (sequence offsets in seg)
  size_t gstride;              // elements between KV heads in either mirror
  int ldp;
  _Float16 *o16;
  int ldo;
  float qscale;  // head_dim^-0.5 * log2(e): scores in base 2
  float *part;   // [split record][piece][query head][32 rows] records of pre_rec_bytes(hd):
                 // o / sum as hd binary16, then max and sum (f32, base 2), pad to 16 bytes
  int n_seg;     // sequences in this launch; block row y is work item y / n_seg of sequence y % n_seg
  PreSeg seg[kPreSegs];
};

// Bytes of one query row's record in the split pieces' workspace: the
// normalised output as hd binary16, the maximum and the sum as f32, padded
// to 16 bytes (hd 64: 144 bytes against 272 for an f32 output).
__host__ __device__ constexpr int pre_rec_bytes(int hd) { return hd * 2 + 16; }


// S = 2 (head_dim <= 64): two wavefronts per query head; the block's two
// halves take the first and the second half of the key tiles, each with its
// own LDS buffers, and their online-softmax states (max, sum, output) are
// merged through LDS at the end.  This doubles the wavefronts a CU runs
// (the grid has about one block per CU) and halves the longest block.
// Groups of 7 add one loader wavefront per half (16 wavefronts at two
// halves, 8 at one): it alone moves the half's K / V^T tiles from global
// memory into LDS, in a loop of its own with the same barriers, so the
// compute wavefronts skip that phase and every SIMD holds the same number
// of wavefronts.
template <int G, int S>
constexpr int prefill_loaders() { return G == 7 ? S : 0; }

template <int HD, int G, int S>
__global__ __launch_bounds__(64 * (G * S + prefill_loaders<G, S>())) void k_attn_prefill(AttnPreP p) {
  constexpr int NL = prefill_loaders<G, S>();  // loader wavefronts (one per half, or none)
  constexpr int KSTEPS = (HD + 15) / 16;
  constexpr int DT = HD >= 32 ? HD / 32 : 1;  // 32-row d tiles of O^T
  constexpr int DV = DT * 32;
  constexpr int KT = kPreKeys;
  constexpr int KP = HD + 8;    // padded LDS row of K (halves)
  constexpr int VP = KT + 8;    // padded LDS row of V^T (halves)
  constexpr int NTHR = 64 * G;       // threads of one half: one wavefront per query head
  constexpr int KCH = KT * HD / 8;   // 16-byte chunks of a K tile (and of a V^T tile)
  constexpr int CPT = (KCH + NTHR - 1) / NTHR;  // chunks per thread
  static_assert(S == 1 || S == 2, "one or two halves");
  constexpr int NF = 2 + 16 * DT;  // merge state per lane: max, sum, output accumulators
  constexpr size_t kTiles = (size_t)S * 2 * (KT * KP + DV * VP) * sizeof(_Float16);
  constexpr size_t kMerge = S == 2 ? (size_t)G * NF * 64 * sizeof(float) : 0;
  // the K / V^T tile buffers, and after the key loop the merge state
  __shared__ __attribute__((aligned(16))) char smem[kTiles > kMerge ? kTiles : kMerge];
  typedef _Float16 KTile[2][KT * KP];
  typedef _Float16 VTile[2][DV * VP];
  KTile *sK = (KTile *)smem;                                      // [S]
  VTile *sV = (VTile *)(smem + (size_t)S * 2 * KT * KP * sizeof(_Float16));  // [S]

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const bool loader = NL > 0 && w >= G * S;  // (wave-uniform)
  const int half = loader ? w - G * S : w / G, hw = loader ? 0 : w - (w / G) * G;
  const int tid = threadIdx.x - half * NTHR, nthr = NTHR;  // index within the half
  // longest work first: with contiguous positions in descending order of
  // key tiles over all items; otherwise the split tiles' two pieces
  // (descending tiles), then the whole tiles (descending)
  // (the KV head is the grid's fastest index, so the dispatch order is
  // longest-first across the KV heads too)
  // (the sequences of the launch interleave, so equal work ranks of all
  // sequences dispatch together)
  const PreSeg &sg = p.seg[blockIdx.y % p.n_seg];
  const int wi = blockIdx.y / p.n_seg;  // work index within the sequence
  const int n_split = sg.n_tiles - sg.split_from;
  if (wi >= sg.n_tiles + n_split) return;  // (a shorter sequence: no work)
  int tile, piece;
  if (sg.p0 >= 0) {
    prefill_item_lpt(sg, wi, tile, piece);
  } else if (wi < 2 * n_split) {
    tile = sg.n_tiles - 1 - wi / 2;
    piece = wi & 1;
  } else {
    tile = sg.split_from - 1 - (wi - 2 * n_split);
    piece = -1;
  }
  const int *pos = p.rows.pos + sg.r0;
  const int g = blockIdx.x;
  const int h = g * p.d.group + blockIdx.z * G + hw;  // (blockIdx.z: G-head share of the group)
  const int r0 = tile * 32;
  const int M = sg.M;
  const int last_row = min(r0 + 31, M - 1);
  const int kmax = pos[last_row];
  const int qrow = r0 + (lane & 31);
  const bool qvalid = qrow < M;
  const int qpos = qvalid ? pos[qrow] : kmax;
  const int qpos_min = pos[r0];  // keys <= this are visible to every row
  const int hi = lane >> 5;
  _Float16(&hK)[2][KT * KP] = sK[half];
  _Float16(&hV)[2][DV * VP] = sV[half];

  if (HD < 32 && NL == 0) {  // d rows HD .. 31 of V^T (never loaded) stay zero
    for (int i = tid; i < 2 * (DV - HD) * VP; i += nthr) {
      const int b = i / ((DV - HD) * VP), j = i - b * (DV - HD) * VP;
      hV[b][HD * VP + j] = (_Float16)0.f;
    }
  }

  if constexpr (NL > 0) {
    if (loader) {
      const _Float16 *kgl = p.k16 + sg.kv_off + (size_t)g * p.gstride;
      const _Float16 *vgl = p.v16t + sg.kv_off + (size_t)g * p.gstride;
      const int ntl = kmax / KT + 1;
      int kbl = 0, kel = ntl;
      if (piece >= 0) {
        const int ph = (ntl + 1) / 2;
        kbl = piece ? ph : 0;
        kel = piece ? ntl : ph;
      }
      const int n0l = (kel - kbl + S - 1) / S;
      const int kt0l = kbl + half * n0l;
      const int cntl = max(0, min(kel, kt0l + n0l) - kt0l);
      // chunk c = lane + 64 i: K at byte 16 c of the tile (its rows of HD
      // halves are contiguous in the mirror); V^T d row c / 8, keys
      // 8 (c % 8) .. +8
      constexpr int LPT = KCH / 64;
      const char *kb8 = (const char *)kgl, *vb8 = (const char *)vgl;
      const unsigned kl = (unsigned)lane * 16u;
      const unsigned vl = (unsigned)(((lane >> 3) * p.ldp + (lane & 7) * 8) * 2);
      const unsigned vstep = (unsigned)(8 * p.ldp * 2);
      h8 lk[LPT], lv[LPT];
      auto lload = [&](int kt) {
        const unsigned kadv = (unsigned)(kt * KT * HD * 2) + kl, vadv = (unsigned)(kt * KT * 2) + vl;
#pragma unroll
        for (int i = 0; i < LPT; ++i) {
          lk[i] = *(const h8 *)(kb8 + (kadv + (unsigned)i * 1024u));
          lv[i] = *(const h8 *)(vb8 + (vadv + (unsigned)i * vstep));
        }
      };
      auto lwrite = [&](int buf) {
#pragma unroll
        for (int i = 0; i < LPT; ++i) {
          const int c = lane + 64 * i;
          const int kk = c / (HD / 8), kc = c - kk * (HD / 8);
          *(h8 *)(&sK[half][buf][kk * KP + kc * 8]) = lk[i];
          *(h8 *)(&sV[half][buf][(c >> 3) * VP + (c & 7) * 8]) = lv[i];
        }
      };
      if (HD < 32) {  // d rows HD .. 31 of V^T (never loaded) stay zero
        for (int i = lane; i < 2 * (DV - HD) * VP; i += 64) {
          const int bb = i / ((DV - HD) * VP), j = i - bb * (DV - HD) * VP;
          sV[half][bb][HD * VP + j] = (_Float16)0.f;
        }
      }
      // the padding chunk of every K row (columns HD .. HD+7, never written
      // by the tile loads): 1, 0, ..., 0
      for (int i = lane; i < 2 * KT; i += 64) {
        h8 one;
#pragma unroll
        for (int j = 0; j < 8; ++j) one[j] = (_Float16)(j == 0 ? 1.f : 0.f);
        *(h8 *)(&sK[half][i / KT][(i % KT) * KP + HD]) = one;
      }
      if (cntl > 0) {
        lload(kt0l);
        lwrite(0);
        if (cntl > 1) lload(kt0l + 1);
      }
      __syncthreads();
      for (int it = 0; it < n0l; ++it) {  // (the compute wavefronts' barriers, one for one)
        if (it + 1 < cntl) lwrite((it + 1) & 1);  // its buffer was last read in it - 1
        if (it + 2 < cntl) lload(kt0l + it + 2);
        __syncthreads();
      }
      if constexpr (S == 2) __syncthreads();  // (the halves' merge)
      return;
    }
  }

  h8 qf[KSTEPS];
  {
    const float *qp = p.q + (size_t)(sg.r0 + (qvalid ? qrow : last_row)) * p.ldq + (size_t)h * HD;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) qf[s][jj] = (_Float16)(qp[s * 16 + hi * 8 + jj] * p.qscale);
  }

  f16x o[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[t][r] = 0.f;
  // Softmax state of the lane's query row.  Scores are taken relative to a
  // reference m_ref (a binary16 value, subtracted on the matrix core by one
  // extra MFMA per 32-key half: a column of ones in K against -m_ref in Q).
  // The reference is raised only when a score exceeds it by more than 10:
  // then to the row's maximum, rescaling O and the sum.  Otherwise a tile
  // takes no cross-lane maximum, rescale or cross-lane sum (the weights
  // 2^(s - m_ref) stay below 2^10, well inside binary16; O and the sum are
  // normalised once at the end, so any reference below the maximum gives
  // the same softmax).  `valid` is false while the row has seen no visible
  // key (m_ref 0).
  float m_ref = 0.f, l_part = 0.f;
  bool valid = false;
  h8 qbias;  // Q-side operand of the reference column: k-slot 0 (lanes 0-31) = -m_ref
#pragma unroll
  for (int j = 0; j < 8; ++j) qbias[j] = (_Float16)0.f;

  const _Float16 *kg = p.k16 + sg.kv_off + (size_t)g * p.gstride;
  const _Float16 *vg = p.v16t + sg.kv_off + (size_t)g * p.gstride;
  const int ntiles = kmax / KT + 1;
  int kb = 0, ke = ntiles;  // this block's key tiles (a split piece takes half)
  if (piece >= 0) {
    const int ph = (ntiles + 1) / 2;
    kb = piece ? ph : 0;
    ke = piece ? ntiles : ph;
  }
  const int n0 = (ke - kb + S - 1) / S;              // tiles of the first half
  const int kt0 = kb + half * n0;                    // this half's first tile
  const int cnt = max(0, min(ke, kt0 + n0) - kt0);   // and its tile count (may be 0)

  // tile loads: chunk c of the K tile is key c / (HD/8), d-chunk c % (HD/8);
  // chunk c of the V^T tile is d c / (KT/8), key-chunk c % (KT/8)
  // (addresses as a block-uniform base plus a 32-bit lane offset: the base
  // stays in scalar registers, so the loop-invariant part costs one vector
  // register per load instead of a 64-bit pointer)
  h8 rk[CPT], rv[CPT];
  const char *kgb = (const char *)kg, *vgb = (const char *)vg;
  unsigned ko[CPT], vo[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = min(tid + i * nthr, KCH - 1);
    const int kk = c / (HD / 8), kc = c - kk * (HD / 8);
    ko[i] = (unsigned)((kk * HD + kc * 8) * 2);
    const int dd = c / (KT / 8), vc = c - dd * (KT / 8);
    vo[i] = (unsigned)((dd * p.ldp + vc * 8) * 2);
  }
  auto gload = [&](int kt) {
    const unsigned kadv = (unsigned)(kt * KT * HD * 2), vadv = (unsigned)(kt * KT * 2);
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * nthr;
      if (c < KCH) {
        rk[i] = *(const h8 *)(kgb + (ko[i] + kadv));
        rv[i] = *(const h8 *)(vgb + (vo[i] + vadv));
      }
    }
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * nthr;
      if (c < KCH) {
        const int kk = c / (HD / 8), kc = c - kk * (HD / 8);
        *(h8 *)(&hK[buf][kk * KP + kc * 8]) = rk[i];
        const int dd = c / (KT / 8), vc = c - dd * (KT / 8);
        *(h8 *)(&hV[buf][dd * VP + vc * 8]) = rv[i];
      }
    }
  };

  // the padding chunk of every K row (columns HD .. HD+7, never written by
  // the tile loads): 1, 0, ..., 0
  if constexpr (NL == 0) {
    for (int i = tid; i < 2 * KT; i += nthr) {
      h8 one;
#pragma unroll
      for (int j = 0; j < 8; ++j) one[j] = (_Float16)(j == 0 ? 1.f : 0.f);
      *(h8 *)(&hK[i / KT][(i % KT) * KP + HD]) = one;
    }
    if (cnt > 0) {
      gload(kt0);
      swrite(0);
      if (cnt > 1) gload(kt0 + 1);
    }
  }
  __syncthreads();
  for (int it = 0; it < n0; ++it) {  // (every half runs n0 iterations: the barriers match)
    const int buf = it & 1;
    const bool live = it < cnt;
    if constexpr (NL == 0) {
      if (it + 1 < cnt) swrite(buf ^ 1);  // its buffer was last read in it - 1
      if (it + 2 < cnt) gload(kt0 + it + 2);
    }
    if (live) {
      const _Float16 *sk = hK[buf];
      const _Float16 *sv = hV[buf];
      const int key0 = (kt0 + it) * KT;
      f16x s[2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[hf][r] = 0.f;
        // the half's fragments read together, then multiplied (one LDS wait
        // instead of one per MFMA; with loader wavefronts the registers are
        // there).  (K side of the reference column: the row's padding chunk,
        // 1 then zeros, read by both lane halves; the upper half's Q side is
        // zero.)
        const _Float16 *kr = sk + (hf * 32 + (lane & 31)) * KP;
        const h8 one = *(const h8 *)(kr + HD);
        h8 a[KSTEPS];
#pragma unroll
        for (int st = 0; st < KSTEPS; ++st) a[st] = *(const h8 *)(kr + st * 16 + hi * 8);
        if (NL > 0) __builtin_amdgcn_sched_barrier(0);
        s[hf] = __builtin_amdgcn_mfma_f32_32x32x16_f16(one, qbias, s[hf], 0, 0, 0);  // - m_ref
#pragma unroll
        for (int st = 0; st < KSTEPS; ++st)
          s[hf] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[st], qf[st], s[hf], 0, 0, 0);
      }
      // causal mask (only tiles that reach past the first row's position)
      if (key0 + KT - 1 > qpos_min) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + hf * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
            if (key > qpos) s[hf][r] = kNegInf;
          }
      }
      // The reference moves when a score of the tile exceeds it by more
      // than 10 (a weight above 2^10), or the row had no visible key yet:
      // then to the row's maximum (rows whose maximum did not move keep it:
      // shift 0, alpha 1), and the tile's scores are shifted to match.
      float mx = kNegInf;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[hf][r]);
      if (__any(!valid || mx > 10.f)) {
        const float mt = max32(mx);  // (relative to m_ref)
        if (mt != kNegInf) {  // (a row with no visible key yet keeps its zero state)
          const float m_abs = fminf(fmaxf(m_ref + (valid ? fmaxf(mt, 0.f) : mt), -60000.f), 60000.f);
          const float m_new = (float)(_Float16)m_abs;
          const float shift = m_new - m_ref;
          const float alpha = valid ? __builtin_amdgcn_exp2f(-shift) : 0.f;
          l_part *= alpha;
#pragma unroll
          for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[t][r] *= alpha;
#pragma unroll
          for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[hf][r] -= shift;
          m_ref = m_new;
          valid = true;
          qbias[0] = (_Float16)(hi == 0 ? -m_new : 0.f);
        }
      }
      // binary16 weights 2^s (the hardware 2^x, v_exp_f32: every argument
      // is <= 10, and results below 2^-126 flush to zero) and the lane's sum
      // of the rounded weights, two at a time in f32 (v_dot2_f32_f16)
      h8 pb[2][2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int r = 0; r < 16; ++r) pb[hf][r >> 3][r & 7] = (_Float16)__builtin_amdgcn_exp2f(s[hf][r]);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int k = 0; k < 8; k += 2)
            l_part = __builtin_amdgcn_fdot2((h2){pb[hf][j][k], pb[hf][j][k + 1]},
                                            (h2){(_Float16)1.f, (_Float16)1.f}, l_part, false);
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const _Float16 *vr = sv + (t * 32 + (lane & 31)) * VP;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const _Float16 *vk = vr + hf * 32;
          const h4 x0 = *(const h4 *)(vk + 4 * hi);
          const h4 x1 = *(const h4 *)(vk + 8 + 4 * hi);
          const h4 x2 = *(const h4 *)(vk + 16 + 4 * hi);
          const h4 x3 = *(const h4 *)(vk + 24 + 4 * hi);
          const h8 a0 = (h8){x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
          const h8 a1 = (h8){x2[0], x2[1], x2[2], x2[3], x3[0], x3[1], x3[2], x3[3]};
          o[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, pb[hf][0], o[t], 0, 0, 0);
          o[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, pb[hf][1], o[t], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }

  float m_run = valid ? m_ref : kNegInf;  // (no visible key: an empty state)
  float l_run = sum32(l_part);
  if constexpr (S == 2) {  // the second half hands its state to the first through LDS
    float *xb = (float *)smem;  // ([hw][field][lane]; the tiles are no longer read)
    if (half == 1) {
      float *x = xb + (size_t)hw * NF * 64 + lane;
      x[0] = m_run;
      x[64] = l_run;
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) x[(2 + t * 16 + r) * 64] = o[t][r];
    }
    __syncthreads();
    if (half == 1) return;
    const float *x = xb + (size_t)hw * NF * 64 + lane;
    const float m1 = x[0], l1 = x[64];
    const float mm = fmaxf(m_run, m1);
    const float mm_sub = mm == kNegInf ? 0.f : mm;  // (no visible key in either half)
    const float a0 = exp2f(m_run - mm_sub), a1 = exp2f(m1 - mm_sub);
    l_run = l_run * a0 + l1 * a1;
    m_run = mm;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[t][r] = o[t][r] * a0 + x[(2 + t * 16 + r) * 64] * a1;
  }

  if (piece >= 0) {  // a split piece: its normalised output, maximum and sum for the merge
    char *pr = (char *)p.part + ((((size_t)(sg.part0 + tile - sg.split_from) * 2 + piece) * p.d.nh + h) * 32 +
                                 (lane & 31)) * pre_rec_bytes(HD);
    const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;  // (a piece with no visible key: zeros)
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d0 = t * 32 + 8 * rq + 4 * hi;
        if (d0 < HD) {
          h4 v = {(_Float16)(o[t][4 * rq + 0] * inv), (_Float16)(o[t][4 * rq + 1] * inv),
                  (_Float16)(o[t][4 * rq + 2] * inv), (_Float16)(o[t][4 * rq + 3] * inv)};
          *(h4 *)(pr + 2 * d0) = v;
        }
      }
    if (hi == 0) *(float2 *)(pr + 2 * HD) = make_float2(m_run, l_run);
    return;
  }
  if (!qvalid) return;
  const float inv_l = 1.0f / l_run;
  _Float16 *orow = p.o16 + (size_t)(sg.r0 + qrow) * p.ldo + (size_t)h * HD;
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int d0 = t * 32 + 8 * rq + 4 * hi;
      if (d0 < HD) {
        h4 v = {(_Float16)(o[t][4 * rq + 0] * inv_l), (_Float16)(o[t][4 * rq + 1] * inv_l),
                (_Float16)(o[t][4 * rq + 2] * inv_l), (_Float16)(o[t][4 * rq + 3] * inv_l)};
        *(h4 *)(orow + d0) = v;
      }
    }
}

// Combines the two pieces of each split query tile: with each piece's
// normalised output o_i / l_i stored, O = (e^(m0-M) o0 + e^(m1-M) o1) /
// (e^(m0-M) l0 + e^(m1-M) l1) is the mean of the two weighted by
// e^(mi-M) li, M the larger maximum (states in base 2).  One block per
// (split tile, query head).
template <int HD>
__global__ __launch_bounds__(256) void k_attn_prefill_merge(AttnPreP p) {
  constexpr int C = HD / 4;                 // 4-wide chunks of a row
  constexpr int IT = (32 * C + 255) / 256;  // chunks per thread
  const int u = blockIdx.x, h = blockIdx.y;  // (u: split record, over all sequences)
  int si = 0;
  while (si + 1 < p.n_seg && u >= p.seg[si + 1].part0) ++si;
  const PreSeg &sg = p.seg[si];
  const int r0 = (sg.split_from + u - sg.part0) * 32;
  const int nq = min(32, sg.M - r0);  // (rows past M come last)
  constexpr int REC = pre_rec_bytes(HD);
  const char *a = (const char *)p.part + (((size_t)u * 2 + 0) * p.d.nh + h) * 32 * REC;
  const char *b = (const char *)p.part + (((size_t)u * 2 + 1) * p.d.nh + h) * 32 * REC;
  // every load first, at clamped rows (a load tied to a condition is waited
  // for on the spot), then the combination
  h4 xa[IT], xb[IT];
  float2 sa[IT], sb[IT];  // (max, sum) of either piece
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int idx = min((int)threadIdx.x + 256 * i, 32 * C - 1);
    const int q = min(idx / C, nq - 1), c = idx % C;
    const char *x = a + q * REC, *y = b + q * REC;
    xa[i] = *(const h4 *)(x + 8 * c);
    xb[i] = *(const h4 *)(y + 8 * c);
    sa[i] = *(const float2 *)(x + 2 * HD);
    sb[i] = *(const float2 *)(y + 2 * HD);
  }
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int idx = (int)threadIdx.x + 256 * i;
    const int q = idx / C, c = idx % C;
    if (idx >= 32 * C || q >= nq) continue;
    const float mm = fmaxf(sa[i].x, sb[i].x);
    const float sub = mm == kNegInf ? 0.f : mm;
    const float w0 = exp2f(sa[i].x - sub) * sa[i].y, w1 = exp2f(sb[i].x - sub) * sb[i].y;
    const float den = w0 + w1;
    h4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (_Float16)(((float)xa[i][e] * w0 + (float)xb[i][e] * w1) / den);
    *(h4 *)(p.o16 + (size_t)(sg.r0 + r0 + q) * p.ldo + (size_t)h * HD + 4 * c) = v;
  }
}

template <int HD, int G>
static void attn_prefill_g(const AttnPreP &p, dim3 grid, hipStream_t st) {
  constexpr int S = HD <= 64 ? 2 : 1;  // (hd 128 needs more registers than 2 halves allow)
  hipLaunchKernelGGL((k_attn_prefill<HD, G, S>), grid, dim3(64 * (G * S + prefill_loaders<G, S>())), 0,
                     st, p);
}

template <int HD>
static void attn_prefill_hd(const AttnPreP &p, int items, int work, int n_split, hipStream_t st) {
  const dim3 grid(p.d.nkv, items * p.n_seg);
  if (n_split > 0) {
    switch (p.d.group) {
      case 7: attn_prefill_g<HD, 7>(p, grid, st); break;
      case 8: attn_prefill_g<HD, 8>(p, grid, st); break;
      case 4: attn_prefill_g<HD, 4>(p, grid, st); break;
      case 2: attn_prefill_g<HD, 2>(p, grid, st); break;
      case 1: attn_prefill_g<HD, 1>(p, grid, st); break;
      case 3: attn_prefill_g<HD, 3>(p, grid, st); break;
      case 5: attn_prefill_g<HD, 5>(p, grid, st); break;
      default: attn_prefill_g<HD, 6>(p, grid, st); break;
    }
    hipLaunchKernelGGL((k_attn_prefill_merge<HD>), dim3(n_split, p.d.nh), dim3(256), 0, st, p);
    return;
  }
  if (p.d.nkv * work < 128) {
    // few query tiles (short prompts): one query head per block, so the
    // group's heads run on separate CUs (each block loads its group's K / V)
    attn_prefill_g<HD, 1>(p, dim3(grid.x, grid.y, p.d.group), st);  // (z: head in the group)
    return;
  }
  switch (p.d.group) {  // the group size is a compile-time constant of the kernel
    case 1: attn_prefill_g<HD, 1>(p, grid, st); break;
    case 2: attn_prefill_g<HD, 2>(p, grid, st); break;
    case 3: attn_prefill_g<HD, 3>(p, grid, st); break;
    case 4: attn_prefill_g<HD, 4>(p, grid, st); break;
    case 5: attn_prefill_g<HD, 5>(p, grid, st); break;
    case 6: attn_prefill_g<HD, 6>(p, grid, st); break;
    case 7: attn_prefill_g<HD, 7>(p, grid, st); break;
    default: attn_prefill_g<HD, 8>(p, grid, st); break;
  }
}

// Up to kPreSegs sequences in one launch.
static void attn_prefill_launch(const Dims &d, int layer, const KVCache &kv, const float *q,
                                int ldq, RowInfo rows, const PrefillSeg *segs, int n,
                                const int *host_pos, const Workspace &ws, _Float16 *o16,
                                int ldo, hipStream_t st) {
  AttnPreP p{};
  p.d = d;
  p.q = q;
  p.ldq = ldq;
  p.rows = rows;
  const size_t b16 = kv.off16(d, layer, 0, 0);
  p.k16 = kv.k16 + b16;
  p.v16t = kv.v16t + b16;
  p.gstride = (size_t)kv.ldp * d.hd;
  p.ldp = kv.ldp;
  p.o16 = o16;
  p.ldo = ldo;
  p.qscale = (1.0f / sqrtf((float)d.hd)) * 1.4426950408889634f;
  p.part = ws.buf;
  p.n_seg = n;
  // Causal balance: with one block per (query tile, KV head) the last tile's
  // block has the most key tiles; tiles with more than a third of the
  // largest count over the launch (and at least 8 key tiles) are split in
  // two, so no block has more than about half of the longest tile's work,
  // and the blocks, dispatched longest first, even out the CUs' finishing
  // times (0.5B 4096-token attention 1.61 -> 1.44 ms per prefill, hd-128
  // 2048 tokens 2.10 -> 1.92 ms, from splitting above half of the largest
  // count with the pieces dispatched before the whole tiles).  Positions
  // increase within a sequence, so the key-tile count grows with the tile
  // index and a sequence's split tiles are its last ones.  With 512 or more
  // blocks (two per CU) the CUs already balance long and short tiles, and
  // the split's merge would only add work (batched 0.5B prefill, 8 x 1024
  // rows per launch: 714 K -> 775 K tok/s without it).
  auto ntiles = [&](const PrefillSeg &g, int t) {
    return host_pos[g.r0 + std::min(32 * t + 31, g.n - 1)] / kPreKeys + 1;
  };
  int total_tiles = 0, kmax = 0;
  for (int i = 0; i < n; ++i) {
    const int T = (segs[i].n + 31) / 32;
    PreSeg &sg = p.seg[i];
    sg.r0 = segs[i].r0;
    sg.M = segs[i].n;
    sg.n_tiles = sg.split_from = T;
    sg.kv_off = kv.off16(d, layer, segs[i].seq, 0) - b16;
    sg.p0 = host_pos[sg.r0];
    for (int r = 1; r < sg.M && sg.p0 >= 0; ++r)
      if (host_pos[sg.r0 + r] != sg.p0 + r) sg.p0 = -1;
    total_tiles += T;
    kmax = std::max(kmax, ntiles(segs[i], T - 1));
  }
  if (total_tiles * d.nkv >= 128 && total_tiles * d.nkv < 512 && kmax >= 8) {
    const int lim = (kmax + 2) / 3;
    int n_split = 0;
    for (int i = 0; i < n; ++i) {
      int sf = p.seg[i].n_tiles;
      while (sf > 0 && ntiles(segs[i], sf - 1) > lim) --sf;
      n_split += p.seg[i].n_tiles - sf;
    }
    const size_t need = (size_t)n_split * 2 * d.nh * 32 * pre_rec_bytes(d.hd);
    if (ws.buf && need <= ws.bytes)
      for (int i = 0; i < n; ++i) {
        int sf = p.seg[i].n_tiles;
        while (sf > 0 && ntiles(segs[i], sf - 1) > lim) --sf;
        p.seg[i].split_from = sf;
      }
  }
  int items = 0, work = 0, n_split = 0;  // (items: the most work items of one sequence)
  for (int i = 0; i < n; ++i) {
    PreSeg &sg = p.seg[i];
    sg.part0 = n_split;
    n_split += sg.n_tiles - sg.split_from;
    items = std::max(items, 2 * sg.n_tiles - sg.split_from);
    work += 2 * sg.n_tiles - sg.split_from;
  }
  switch (d.hd) {
    case 16: attn_prefill_hd<16>(p, items, work, n_split, st); break;
    case 64: attn_prefill_hd<64>(p, items, work, n_split, st); break;
    default: attn_prefill_hd<128>(p, items, work, n_split, st); break;
  }
}

void attn_prefill(const Dims &d, int layer, const KVCache &kv, const float *q, int ldq,
                  RowInfo rows, const PrefillSeg *segs, int n_segs, const int *host_pos,
                  const Workspace &ws, _Float16 *o16, int ldo, hipStream_t st) {
  for (int i = 0; i < n_segs; i += kPreSegs)
    attn_prefill_launch(d, layer, kv, q, ldq, rows, segs + i, std::min(kPreSegs, n_segs - i),
                        host_pos, ws, o16, ldo, st);
}

}  // namespace q2
