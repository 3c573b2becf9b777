// C ABI of the MI355X Qwen2 decoder forward pass: context, device weight
// store, KV cache, scratch and the per-call launch sequence.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <list>
#include <string>
#include <tuple>
#include <utility>
#include <vector>

#include "../../include/qwen2.h"
#include "q2_kernels.h"
#include "validate.h"

using q2::Dims;
using q2::LayerW;

namespace {

constexpr int kRing = 4;          // pinned staging slots for per-call row data
constexpr int kGemvRows = 8;      // rows up to this use the f32 GEMV path
constexpr int kMaxPassRows = 4096;   // rows per prefill pass of one sequence
constexpr int kMaxBatchRows = 8192;  // rows per pass of a multi-sequence context
constexpr int kProfMax = 16384;     // timed launches between two reads
constexpr size_t kSlotBytes = 64;   // pointer slots at the head of a staged call
constexpr size_t kSplitKBytes = 64ull << 20;  // split-K partial sums (large-M residual GEMMs: <= 256 x 256 x 256 x 4 B)
constexpr size_t kMaxGraphs = 32;   // captured decode steps kept per context
using GraphKey = std::tuple<int, int, int>;  // (rows, attention chunks, slot of a one-row step)

thread_local std::string g_load_error;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

struct qwen2_ctx {
  qwen2_hparams hp{};
  Dims d{};
  int device = 0;
  // weight store
  char *warena = nullptr;
  size_t warena_bytes = 0;
  const uint16_t *tok_embd = nullptr, *lm_head = nullptr;
  const float *out_norm = nullptr;
  std::vector<LayerW> layers;
  uint64_t w_f16 = 0, w_f32 = 0;
  // KV cache and RoPE table
  float *kc = nullptr, *vc = nullptr;
  _Float16 *kc16 = nullptr, *vc16t = nullptr;  // binary16 mirror (prefill attention)
  int ldp = 0;                                 // mirror positions: n_ctx rounded up to 64
  size_t kv_elems = 0;
  float *rope_cos = nullptr, *rope_sin = nullptr;
  // scratch
  char *sarena = nullptr;
  size_t sarena_bytes = 0;
  int max_rows = 0;   // rows per prefill pass
  int rows_cap = 0;   // rows of the activation buffers: max(max_rows, n_seq)
  int dec_rows = 0;   // rows of the GEMV / decode-attention buffers: max(n_seq, 8)
  float *h = nullptr, *q32 = nullptr, *o32 = nullptr, *a32 = nullptr, *normed = nullptr;
  _Float16 *x16 = nullptr, *a16 = nullptr;
  // Device copy of the per-call block: pointer slots (tokens, logits, argmax)
  // then the row data (prefill: tokens | positions | seqs; decode:
  // positions | seqs).  Kernels read everything per call from here, so a
  // captured decode graph serves every call of its batch size.
  char *io = nullptr;
  size_t io_cap = 0;  // int entries per field
  q2::AttnPartials part{};
  q2::Workspace splitk{};  // split-K partial sums of the small-M GEMMs
  unsigned long long *best = nullptr;
  unsigned int *bad_flag = nullptr;
  int *stop_ids = nullptr;     // [1 + kMaxStopIds]: count, then the ids
  unsigned *stop_pos = nullptr;  // [n_seq] latched stop positions (~0u: none)
  float2 *prob_part = nullptr;   // [dec_rows][kProbBlocks] softmax partials
  // captured decode steps, keyed by (batch size, attention chunks, slot of
  // a one-row step), least recently used first; at most kMaxGraphs live
  std::list<std::pair<GraphKey, hipGraphExec_t>> graphs;
  hipStream_t cap_stream = nullptr;  // captures only (never runs work)
  bool use_graphs = true;
  // pinned staging ring
  char *pinned = nullptr;
  hipEvent_t ev[kRing] = {};
  int ring = 0;
  // last read-out rows
  const float *last_h = nullptr;
  int last_rows = 0;
  // per-op timing (qwen2_prof_*)
  uint32_t prof_mask = 0;
  std::vector<hipEvent_t> prof_ev;  // 2 per timed launch
  int prof_used = 0;
  std::vector<std::pair<int, int>> prof_rec;  // (op, event pair)
  // debug checks (QWEN2_DEBUG_CHECKS=1 at load): the call's slot mask
  // [n_seq][n_ctx] and the results [8]: hash before, hash after, first
  // non-finite K word, V word, logit, hidden value (~0: none), 2 spare
  bool debug = false;
  unsigned char *dbg_mask = nullptr;
  unsigned long long *dbg = nullptr;
  std::vector<unsigned char> dbg_host;
  std::string err;
};

namespace {

}  // namespace

void q2::set_static_error(const std::string &msg) { g_load_error = msg; }

namespace {

int set_err(qwen2_ctx *c, int code, const std::string &m) {
  if (c) c->err = m;
  else g_load_error = m;
  return code;
}

#define HIP_TRY(ctx, expr)                                                                \
  do {                                                                                    \
    hipError_t e_ = (expr);                                                               \
    if (e_ != hipSuccess)                                                                 \
      return set_err(ctx, e_ == hipErrorOutOfMemory ? QWEN2_E_OOM : QWEN2_E_HIP,          \
                     std::string(#expr) + ": " + hipGetErrorString(e_));                  \
  } while (0)

void release(qwen2_ctx *c) {
  if (!c) return;
  (void)hipDeviceSynchronize();
  if (c->warena) (void)hipFree(c->warena);
  if (c->kc) (void)hipFree(c->kc);
  if (c->vc) (void)hipFree(c->vc);
  if (c->kc16) (void)hipFree(c->kc16);
  if (c->vc16t) (void)hipFree(c->vc16t);
  if (c->rope_cos) (void)hipFree(c->rope_cos);
  if (c->sarena) (void)hipFree(c->sarena);
  if (c->dbg_mask) (void)hipFree(c->dbg_mask);
  if (c->dbg) (void)hipFree(c->dbg);
  if (c->pinned) (void)hipHostFree(c->pinned);
  for (auto &e : c->ev)
    if (e) (void)hipEventDestroy(e);
  for (auto &e : c->prof_ev) (void)hipEventDestroy(e);
  for (auto &g : c->graphs) (void)hipGraphExecDestroy(g.second);
  if (c->cap_stream) (void)hipStreamDestroy(c->cap_stream);
  delete c;
}

// Packs the fused QKV rows.  The kernels rotate packed row pair (2j, 2j+1)
// of a head by RoPE angle j and write the pair to dimensions j and j + hd/2
// of the q row or KV slot.  NonInterleaved (and every v head): packed rows
// (2j, 2j+1) = natural rows (j, j + hd/2), so dimensions keep their order.
// Interleaved q and k heads: packed rows (2j, 2j+1) = natural rows (2j,
// 2j+1), the pair the Interleaved style rotates by angle j; q and k then
// hold the same permutation of their dimensions (2j -> j, 2j+1 -> j + hd/2),
// which leaves every q.k product, and so the attention, unchanged.  The
// cache's K copies (qwen2_kv_read / kv_write) undo and apply it.
template <typename T>
void pack_qkv(const qwen2_hparams &hp, const T *q, const T *k, const T *v, size_t rowlen,
              std::vector<T> &out) {
  const int hd = hp.head_dim, half = hd / 2;
  const int nh = hp.n_head, nkv = hp.n_head_kv;
  out.assign((size_t)(nh + 2 * nkv) * hd * rowlen, T(0));
  size_t dst_row = 0;
  auto put_heads = [&](const T *src, int heads, bool interleaved) {
    for (int hh = 0; hh < heads; ++hh)
      for (int j = 0; j < half; ++j) {
        for (int part = 0; part < 2; ++part) {
          const int dim = interleaved ? 2 * j + part : j + part * half;
          const size_t srow = (size_t)hh * hd + dim;
          memcpy(&out[dst_row * rowlen], src + srow * rowlen, rowlen * sizeof(T));
          ++dst_row;
        }
      }
  };
  const bool il = hp.rope_style == 1;
  put_heads(q, nh, il);
  put_heads(k, nkv, il);
  put_heads(v, nkv, false);
}

}  // namespace

extern "C" {

int qwen2_load(const qwen2_hparams *hp, const qwen2_weights *w, void *stream, qwen2_ctx **out) {
  if (!out) return set_err(nullptr, QWEN2_E_ARG, "null output pointer");
  *out = nullptr;
  std::string msg;
  int rc = q2::check_hparams(hp, &msg);
  if (rc) return set_err(nullptr, rc, msg);
  if (!w || !w->tok_embd || !w->out_norm || !w->layers || (!hp->tied && !w->lm_head))
    return set_err(nullptr, QWEN2_E_ARG, "missing weight pointer");
  for (int l = 0; l < hp->n_layer; ++l) {
    const qwen2_layer_weights &L = w->layers[l];
    if (!L.attn_norm || !L.bq || !L.bk || !L.bv || !L.ffn_norm || !L.wq || !L.wk || !L.wv ||
        !L.wo || !L.w_gate || !L.w_up || !L.w_down)
      return set_err(nullptr, QWEN2_E_ARG, "missing weight pointer in layer " + std::to_string(l));
  }
  hipStream_t st = (hipStream_t)stream;

  qwen2_ctx *c = new qwen2_ctx();
  c->hp = *hp;
  Dims &d = c->d;
  d.L = hp->n_layer;
  d.H = hp->n_embd;
  d.nh = hp->n_head;
  d.nkv = hp->n_head_kv;
  d.hd = hp->head_dim;
  d.group = d.nh / d.nkv;
  d.I = hp->n_ff;
  d.I_pad = (d.I + 63) / 64 * 64;
  d.V = hp->n_vocab;
  d.n_ctx = hp->n_ctx;
  d.n_seq = hp->n_seq;
  d.nqkv = (d.nh + 2 * d.nkv) * d.hd;

  auto fail = [&](int code) {
    std::string m = c->err;
    release(c);
    return set_err(nullptr, code, m);
  };
#define LTRY(expr)                    \
  do {                                \
    int r_ = (expr);                  \
    if (r_) return fail(r_);          \
  } while (0)

  LTRY([&]() -> int { HIP_TRY(c, hipGetDevice(&c->device)); return 0; }());

  // ---- weight store layout
  const size_t H = d.H, V = d.V, I = d.I, Ip = d.I_pad, nq = d.nqkv, nhd = (size_t)d.nh * d.hd;
  struct Slot { size_t off, bytes; };
  size_t cur = 0;
  auto take = [&](size_t bytes) { Slot s{cur, bytes}; cur = align256(cur + bytes); return s; };
  Slot s_emb = take(V * H * 2);
  Slot s_lm = hp->tied ? s_emb : take(V * H * 2);
  Slot s_onorm = take(H * 4);
  std::vector<Slot> s_l(7 * d.L);
  for (int l = 0; l < d.L; ++l) {
    s_l[7 * l + 0] = take(H * 4);        // attn_norm
    s_l[7 * l + 1] = take(H * 4);        // ffn_norm
    s_l[7 * l + 2] = take(nq * 4);       // bqkv
    s_l[7 * l + 3] = take(nq * H * 2);   // wqkv
    s_l[7 * l + 4] = take(H * nhd * 2);  // wo
    s_l[7 * l + 5] = take(2 * Ip * H * 2);  // wgu
    s_l[7 * l + 6] = take(H * Ip * 2);   // wd
  }
  c->warena_bytes = cur;
  c->w_f16 = (uint64_t)(V * H * (hp->tied ? 1 : 2) +
                        d.L * (nq * H + H * nhd + 3 * I * H)) * 2;
  c->w_f32 = (uint64_t)(H + d.L * (2 * H + nq)) * 4;
  LTRY([&]() -> int { HIP_TRY(c, hipMalloc(&c->warena, c->warena_bytes)); return 0; }());
  char *A = c->warena;
  auto put = [&](const Slot &s, const void *src) -> int {
    HIP_TRY(c, hipMemcpy(A + s.off, src, s.bytes, hipMemcpyHostToDevice));
    return 0;
  };
  LTRY(put(s_emb, w->tok_embd));
  if (!hp->tied) LTRY(put(s_lm, w->lm_head));
  LTRY(put(s_onorm, w->out_norm));
  c->tok_embd = (const uint16_t *)(A + s_emb.off);
  c->lm_head = (const uint16_t *)(A + s_lm.off);
  c->out_norm = (const float *)(A + s_onorm.off);
  {
    std::vector<uint16_t> tmp16;
    std::vector<float> tmp32;
    for (int l = 0; l < d.L; ++l) {
      const qwen2_layer_weights &L = w->layers[l];
      const Slot *s = &s_l[7 * l];
      LTRY(put(s[0], L.attn_norm));
      LTRY(put(s[1], L.ffn_norm));
      pack_qkv<float>(*hp, L.bq, L.bk, L.bv, 1, tmp32);
      LTRY(put(s[2], tmp32.data()));
      pack_qkv<uint16_t>(*hp, L.wq, L.wk, L.wv, H, tmp16);
      LTRY(put(s[3], tmp16.data()));
      LTRY(put(s[4], L.wo));
      tmp16.assign(2 * Ip * H, 0);
      for (size_t i = 0; i < I; ++i) {
        memcpy(&tmp16[(2 * i) * H], L.w_gate + i * H, H * 2);
        memcpy(&tmp16[(2 * i + 1) * H], L.w_up + i * H, H * 2);
      }
      LTRY(put(s[5], tmp16.data()));
      tmp16.assign(H * Ip, 0);
      for (size_t r = 0; r < H; ++r) memcpy(&tmp16[r * Ip], L.w_down + r * I, I * 2);
      LTRY(put(s[6], tmp16.data()));
      LayerW lw;
      lw.attn_norm = (const float *)(A + s[0].off);
      lw.ffn_norm = (const float *)(A + s[1].off);
      lw.bqkv = (const float *)(A + s[2].off);
      lw.wqkv = (const uint16_t *)(A + s[3].off);
      lw.wo = (const uint16_t *)(A + s[4].off);
      lw.wgu = (const uint16_t *)(A + s[5].off);
      lw.wd = (const uint16_t *)(A + s[6].off);
      c->layers.push_back(lw);
    }
  }

  // ---- KV cache (zero-filled: slots never written read as zero)
  c->kv_elems = (size_t)d.L * d.n_seq * d.nkv * d.n_ctx * d.hd;
  LTRY([&]() -> int {
    HIP_TRY(c, hipMalloc(&c->kc, c->kv_elems * 4));
    HIP_TRY(c, hipMalloc(&c->vc, c->kv_elems * 4));
    HIP_TRY(c, hipMemset(c->kc, 0, c->kv_elems * 4));
    HIP_TRY(c, hipMemset(c->vc, 0, c->kv_elems * 4));
    c->ldp = (d.n_ctx + 63) / 64 * 64;
    const size_t e16 = (size_t)d.L * d.n_seq * d.nkv * c->ldp * d.hd;
    HIP_TRY(c, hipMalloc(&c->kc16, e16 * 2));
    HIP_TRY(c, hipMalloc(&c->vc16t, e16 * 2));
    HIP_TRY(c, hipMemset(c->kc16, 0, e16 * 2));
    HIP_TRY(c, hipMemset(c->vc16t, 0, e16 * 2));
    return 0;
  }());

  // ---- RoPE table: angle = pos * freq_scale * theta^(-2j/hd), computed in
  // double and rounded to float once.
  {
    const int half = d.hd / 2;
    std::vector<float> cs((size_t)d.n_ctx * half), sn((size_t)d.n_ctx * half);
    for (int p = 0; p < d.n_ctx; ++p)
      for (int j = 0; j < half; ++j) {
        const double inv = pow((double)hp->rope_theta, -2.0 * j / d.hd);
        const double ang = (double)p * (double)hp->rope_freq_scale * inv;
        cs[(size_t)p * half + j] = (float)cos(ang);
        sn[(size_t)p * half + j] = (float)sin(ang);
      }
    LTRY([&]() -> int {
      HIP_TRY(c, hipMalloc(&c->rope_cos, 2 * cs.size() * 4));
      c->rope_sin = c->rope_cos + cs.size();
      HIP_TRY(c, hipMemcpy(c->rope_cos, cs.data(), cs.size() * 4, hipMemcpyHostToDevice));
      HIP_TRY(c, hipMemcpy(c->rope_sin, sn.data(), sn.size() * 4, hipMemcpyHostToDevice));
      return 0;
    }());
  }

  // ---- scratch
  // one sequence never has more than n_ctx rows; a batch of several may
  c->max_rows = d.n_seq > 1 ? kMaxBatchRows : std::min(d.n_ctx, kMaxPassRows);
  c->rows_cap = std::max(c->max_rows, d.n_seq);
  c->dec_rows = std::max(d.n_seq, kGemvRows);
  c->part.n_chunks = (d.n_ctx + q2::kChunkKeys - 1) / q2::kChunkKeys;
  c->io_cap = (size_t)std::max(d.n_ctx, c->max_rows + d.n_seq);
  const char *ng = getenv("QWEN2_NO_GRAPH");
  c->use_graphs = !(ng && ng[0] == '1');
  const char *dc = getenv("QWEN2_DEBUG_CHECKS");
  c->debug = dc && dc[0] == '1';
  if (c->debug) {
    c->dbg_host.assign((size_t)d.n_seq * d.n_ctx, 0);
    LTRY([&]() -> int {
      HIP_TRY(c, hipMalloc(&c->dbg_mask, c->dbg_host.size()));
      HIP_TRY(c, hipMalloc(&c->dbg, 8 * sizeof(unsigned long long)));
      return 0;
    }());
  }
  {
    const size_t R = c->rows_cap, D = c->dec_rows;
    cur = 0;
    Slot s_h = take(R * H * 4), s_q = take(R * nhd * 4), s_x16 = take(R * H * 2),
         s_a16 = take(R * Ip * 2), s_o32 = take(D * nhd * 4), s_a32 = take(D * Ip * 4),
         s_norm = take(D * H * 4), s_io = take(kSlotBytes + 3 * c->io_cap * 4),
         s_part = take((size_t)D * d.nkv * c->part.n_chunks * q2::attn_rec_floats(d.group, d.hd) * 4),
         s_best = take(D * 8), s_bad = take(4), s_splitk = take(kSplitKBytes),
         s_stop = take((1 + q2::kMaxStopIds) * 4), s_stop_pos = take((size_t)d.n_seq * 4),
         s_prob = take(D * q2::kProbBlocks * sizeof(float2));
    c->sarena_bytes = cur;
    LTRY([&]() -> int {
      HIP_TRY(c, hipMalloc(&c->sarena, c->sarena_bytes));
      HIP_TRY(c, hipMemset(c->sarena, 0, c->sarena_bytes));
      HIP_TRY(c, hipMemset(c->sarena + s_stop_pos.off, 0xFF, (size_t)d.n_seq * 4));
      return 0;
    }());
    char *S = c->sarena;
    c->h = (float *)(S + s_h.off);
    c->q32 = (float *)(S + s_q.off);
    c->x16 = (_Float16 *)(S + s_x16.off);
    c->a16 = (_Float16 *)(S + s_a16.off);
    c->o32 = (float *)(S + s_o32.off);
    c->a32 = (float *)(S + s_a32.off);
    c->normed = (float *)(S + s_norm.off);
    c->io = S + s_io.off;
    c->part.buf = (float *)(S + s_part.off);
    c->best = (unsigned long long *)(S + s_best.off);
    c->splitk = q2::Workspace{(float *)(S + s_splitk.off), kSplitKBytes};
    c->bad_flag = (unsigned *)(S + s_bad.off);
    c->stop_ids = (int *)(S + s_stop.off);
    c->stop_pos = (unsigned *)(S + s_stop_pos.off);
    c->prob_part = (float2 *)(S + s_prob.off);
  }
  LTRY([&]() -> int {
    HIP_TRY(c, hipHostMalloc((void **)&c->pinned, kRing * (kSlotBytes + 3 * c->io_cap * 4),
                             hipHostMallocDefault));
    for (auto &e : c->ev) HIP_TRY(c, hipEventCreateWithFlags(&e, hipEventDisableTiming));
    HIP_TRY(c, hipStreamCreateWithFlags(&c->cap_stream, hipStreamNonBlocking));
    HIP_TRY(c, hipStreamSynchronize(st));
    HIP_TRY(c, hipDeviceSynchronize());
    return 0;
  }());
#undef LTRY
  *out = c;
  return QWEN2_OK;
}

}  // extern "C"

namespace {

// Pointer slots at the head of the staged per-call block.
struct CallSlots {
  const int *tokens;
  float *logits;
  int *argmax;
};

// Writes the call block (pointer slots + `nf` int32 fields of n entries)
// into the next pinned ring slot and copies it to the device block; returns
// device addresses of the fields.
int stage_call(qwen2_ctx *c, hipStream_t st, const CallSlots &slots, int n, int nf,
               const int32_t *const *fields, int **dev_fields) {
  const int slot = c->ring;
  c->ring = (c->ring + 1) % kRing;
  HIP_TRY(c, hipEventSynchronize(c->ev[slot]));
  char *hb = c->pinned + (size_t)slot * (kSlotBytes + 3 * c->io_cap * 4);
  memcpy(hb, &slots, sizeof slots);
  int32_t *hi = (int32_t *)(hb + kSlotBytes);
  for (int f = 0; f < nf; ++f) {
    memcpy(hi + (size_t)f * n, fields[f], (size_t)n * 4);
    dev_fields[f] = (int *)(c->io + kSlotBytes) + (size_t)f * n;
  }
  HIP_TRY(c, hipMemcpyAsync(c->io, hb, kSlotBytes + (size_t)nf * n * 4, hipMemcpyHostToDevice, st));
  HIP_TRY(c, hipEventRecord(c->ev[slot], st));
  return QWEN2_OK;
}

const CallSlots *dev_slots(qwen2_ctx *c) { return (const CallSlots *)c->io; }

q2::KVCache kv_of(const qwen2_ctx *c) { return q2::KVCache{c->kc, c->vc, c->kc16, c->vc16t, c->ldp}; }

q2::ArgmaxEpi argmax_epi(qwen2_ctx *c, q2::RowInfo rows) {
  const CallSlots *ds = dev_slots(c);
  return q2::ArgmaxEpi{(float *const *)&ds->logits, c->best, (int *const *)&ds->argmax, rows,
                       c->stop_ids, c->stop_pos};
}

int chunks_for(int max_pos) { return (max_pos + q2::kChunkKeys) / q2::kChunkKeys; }

// Brackets one op launch with two events when that op kind is being timed.
struct OpTimer {
  qwen2_ctx *c;
  int op, idx = -1;
  hipStream_t st;
  OpTimer(qwen2_ctx *c_, int op_, hipStream_t st_) : c(c_), op(op_), st(st_) {
    if ((c->prof_mask >> op) & 1u && c->prof_used < kProfMax) {
      idx = c->prof_used++;
      (void)hipEventRecord(c->prof_ev[2 * idx], st);
    }
  }
  ~OpTimer() {
    if (idx >= 0) {
      (void)hipEventRecord(c->prof_ev[2 * idx + 1], st);
      c->prof_rec.emplace_back(op, idx);
    }
  }
};
#define TIMED(op, call)             \
  do {                              \
    OpTimer t_(c, (op), st);        \
    call;                           \
  } while (0)

// Attention then WO + residual on the GEMV path (M <= 8 rows, q in q32,
// output added to rows h).  seq1: the sequence slot of a one-row call
// (unused otherwise).  Short contexts run one fused kernel (head
// attention times a WO slice, atomically added to h); longer ones run the
// chunked attention, then one kernel that merges its chunk records and
// multiplies by WO the same way.
void attn_wo_gemv(qwen2_ctx *c, int l, const float *q, q2::RowInfo rows, int M, int n_chunks,
                  int seq1, float *h, hipStream_t st) {
  const Dims &d = c->d;
  const LayerW &w = c->layers[l];
  const int nhd = d.nh * d.hd;
  const q2::KVCache kv = kv_of(c);
  if (n_chunks * q2::kChunkKeys <= q2::kFusedKeys) {
    // one row: its slot and a key bound past its position, from the host
    const int nk1 = std::min(n_chunks * q2::kChunkKeys, d.n_ctx);
    const uint16_t *next_qkv = l + 1 < d.L ? c->layers[l + 1].wqkv : nullptr;
    TIMED(QWEN2_OP_ATTN, q2::attn_wo_fused(d, l, kv, q, nhd, rows, M, seq1, nk1, w.wo, h, d.H,
                                           w.wd, next_qkv, st));
    return;
  }
  TIMED(QWEN2_OP_ATTN, q2::attn_decode(d, l, kv, q, nhd, rows, M, n_chunks, false, c->part,
                                       nullptr, nullptr, nhd, st));
  TIMED(QWEN2_OP_WO, q2::merge_wo(d, c->part, rows, M, w.wo, h, d.H, st));
}

q2::QkvEpi qkv_epi(qwen2_ctx *c, int l, const int *pos, const int *seq) {
  q2::QkvEpi e;
  e.bias = c->layers[l].bqkv;
  e.q = c->q32;
  e.ldq = c->d.nh * c->d.hd;
  e.kv = kv_of(c);
  e.layer = l;
  e.rows = q2::RowInfo{pos, seq};
  e.rope = q2::RopeTable{c->rope_cos, c->rope_sin};
  return e;
}

// The last layer of a prefill pass after its K/V are stored: only the last
// row goes on (attention, WO, FFN, final norm, lm_head, argmax).
void tail_row(qwen2_ctx *c, int r, const int *pos, const int *seq, int last_pos, int host_seq,
              hipStream_t st) {
  const Dims &d = c->d;
  const int l = d.L - 1;
  const LayerW &w = c->layers[l];
  const int nhd = d.nh * d.hd;
  float *hr = c->h + (size_t)r * d.H;
  attn_wo_gemv(c, l, c->q32 + (size_t)r * nhd, q2::RowInfo{pos + r, seq + r}, 1,
               chunks_for(last_pos), host_seq, hr, st);
  TIMED(QWEN2_OP_GATEUP, q2::gemv_swiglu(d, w, hr, 1, c->a32, d.I_pad, c->hp.rms_eps, c->normed, st));
  TIMED(QWEN2_OP_DOWN, q2::gemv_resid(w.wd, d.H, d.I_pad, c->a32, d.I_pad, 1, hr, d.H, st));
  TIMED(QWEN2_OP_LMHEAD, q2::gemv_lmhead(d, c->lm_head, c->out_norm, hr, 1, c->normed,
                                         argmax_epi(c, q2::RowInfo{pos + r, seq + r}),
                                         c->hp.rms_eps, st));
  c->last_h = hr;
  c->last_rows = 1;
}

// A run of rows of one sequence inside a prefill pass.
using Seg = q2::PrefillSeg;

// One pass of at most max_rows rows (runs of rows of one or more sequences,
// `segs`), up to and including the last layer's Q/K/V: every row's K/V is
// then stored and, with the last layer's input norm having folded every
// pending partial sum, h and q32 hold each row's last-layer input and query.
void prefill_pass(qwen2_ctx *c, int M, int off, const int *pos, const int *seq,
                  const std::vector<Seg> &segs, const int32_t *host_pos, hipStream_t st) {
  const Dims &d = c->d;
  const float eps = c->hp.rms_eps;
  const int nhd = d.nh * d.hd;
  const q2::KVCache kv = kv_of(c);
  const q2::RowInfo rows{pos, seq};
  TIMED(QWEN2_OP_EMBED, q2::embed_rows(c->tok_embd, d.H, d.V, &dev_slots(c)->tokens, off, M,
                                       c->h, c->bad_flag, st));
  int max_pos = 0;
  for (const Seg &g : segs) max_pos = std::max(max_pos, (int)host_pos[g.r0 + g.n - 1]);
  const int n_chunks = chunks_for(max_pos);
  const bool gemv = M <= kGemvRows;
  int pending = 0;  // split-K partial sums of the last residual GEMM not yet in h
  for (int l = 0; l < d.L; ++l) {
    const LayerW &w = c->layers[l];
    const q2::QkvEpi e = qkv_epi(c, l, pos, seq);
    if (gemv) {
      TIMED(QWEN2_OP_QKV, q2::gemv_qkv(d, w, c->h, M, e, eps, c->normed, st));
    } else if (pending == 0 && q2::qkv_fuses_norm(d, M, c->splitk)) {
      TIMED(QWEN2_OP_QKV, q2::gemm_qkv_normed(d, w, c->h, d.H, M, eps, e, st));
    } else {
      TIMED(QWEN2_OP_NORM, q2::rmsnorm_rows_f16(c->h, d.H, w.attn_norm, d.H, M, eps, c->x16, d.H,
                                                nullptr, c->splitk.buf, pending, st));
      pending = 0;
      TIMED(QWEN2_OP_QKV, q2::gemm_qkv(d, w, c->x16, d.H, M, e, c->splitk, st));
    }
    if (l == d.L - 1) break;  // the last layer goes on for read-out rows only
    if (gemv) {
      attn_wo_gemv(c, l, c->q32, rows, M, n_chunks, segs[0].seq, c->h, st);
      TIMED(QWEN2_OP_GATEUP, q2::gemv_swiglu(d, w, c->h, M, c->a32, d.I_pad, eps, c->normed, st));
      TIMED(QWEN2_OP_DOWN, q2::gemv_resid(w.wd, d.H, d.I_pad, c->a32, d.I_pad, M, c->h, d.H, st));
    } else {
      TIMED(QWEN2_OP_ATTN, q2::attn_prefill(d, l, kv, c->q32, nhd, rows, segs.data(),
                                            (int)segs.size(), host_pos, c->splitk, c->x16, nhd,
                                            st));
      TIMED(QWEN2_OP_WO, pending = q2::gemm_resid(w.wo, d.H, nhd, c->x16, nhd, M, c->h, d.H,
                                                  c->splitk, st));
      TIMED(QWEN2_OP_NORM, q2::rmsnorm_rows_f16(c->h, d.H, w.ffn_norm, d.H, M, eps, c->x16, d.H,
                                                nullptr, c->splitk.buf, pending, st));
      TIMED(QWEN2_OP_GATEUP, q2::gemm_swiglu(d, w, c->x16, d.H, M, c->a16, d.I_pad, c->splitk, st));
      TIMED(QWEN2_OP_DOWN, pending = q2::gemm_resid(w.wd, d.H, d.I_pad, c->a16, d.I_pad, M, c->h,
                                                    d.H, c->splitk, st));
    }
  }
}

// Attention onwards of layer l for B rows of independent positions (their
// K/V stored, queries in q32 rows 0..B-1, residual stream in h rows
// 0..B-1; seq1 = the slot of a one-row call).  Returns the split-K
// partial-sum sets left pending in h.
int rows_rest(qwen2_ctx *c, int l, int B, int n_chunks, q2::RowInfo rows, int seq1,
              hipStream_t st) {
  const Dims &d = c->d;
  const float eps = c->hp.rms_eps;
  const int nhd = d.nh * d.hd;
  const LayerW &w = c->layers[l];
  if (B <= kGemvRows) {
    attn_wo_gemv(c, l, c->q32, rows, B, n_chunks, seq1, c->h, st);
    TIMED(QWEN2_OP_GATEUP, q2::gemv_swiglu(d, w, c->h, B, c->a32, d.I_pad, eps, c->normed, st));
    TIMED(QWEN2_OP_DOWN, q2::gemv_resid(w.wd, d.H, d.I_pad, c->a32, d.I_pad, B, c->h, d.H, st));
    return 0;
  }
  int pending;
  TIMED(QWEN2_OP_ATTN, q2::attn_decode(d, l, kv_of(c), c->q32, nhd, rows, B, n_chunks, true,
                                       c->part, nullptr, c->x16, nhd, st));
  TIMED(QWEN2_OP_WO, pending = q2::gemm_resid(w.wo, d.H, nhd, c->x16, nhd, B, c->h, d.H,
                                              c->splitk, st));
  TIMED(QWEN2_OP_NORM, q2::rmsnorm_rows_f16(c->h, d.H, w.ffn_norm, d.H, B, eps, c->x16, d.H,
                                            nullptr, c->splitk.buf, pending, st));
  TIMED(QWEN2_OP_GATEUP, q2::gemm_swiglu(d, w, c->x16, d.H, B, c->a16, d.I_pad, c->splitk, st));
  TIMED(QWEN2_OP_DOWN, pending = q2::gemm_resid(w.wd, d.H, d.I_pad, c->a16, d.I_pad, B, c->h,
                                                d.H, c->splitk, st));
  return pending;
}

// Final norm, lm_head and argmax of h rows 0..B-1 into the staged slots.
void rows_head(qwen2_ctx *c, int B, q2::RowInfo rows, int pending, hipStream_t st) {
  const Dims &d = c->d;
  const float eps = c->hp.rms_eps;
  if (B <= kGemvRows) {
    TIMED(QWEN2_OP_LMHEAD, q2::gemv_lmhead(d, c->lm_head, c->out_norm, c->h, B, c->normed,
                                           argmax_epi(c, rows), eps, st));
  } else {
    TIMED(QWEN2_OP_NORM, q2::rmsnorm_rows_f16(c->h, d.H, c->out_norm, d.H, B, eps, c->x16, d.H,
                                              c->normed, c->splitk.buf, pending, st));
    TIMED(QWEN2_OP_LMHEAD, q2::gemm_lmhead(d, c->lm_head, c->x16, d.H, B, argmax_epi(c, rows),
                                           st));
  }
}

// Every kernel of one decode step for B rows (replayed from a graph).
void decode_launches(qwen2_ctx *c, int B, int n_chunks, const int *dpos, const int *dseq,
                     int seq1, hipStream_t st) {
  const Dims &d = c->d;
  const float eps = c->hp.rms_eps;
  const q2::RowInfo rows{dpos, dseq};
  // (one row: the gather is folded into the first QKV projection)
  const q2::EmbedSrc emb{c->tok_embd, d.V, &dev_slots(c)->tokens, 0, c->bad_flag};
  const bool emb_fused = q2::gemv_qkv_embeds(d, B);
  if (!emb_fused)
    TIMED(QWEN2_OP_EMBED, q2::embed_rows(c->tok_embd, d.H, d.V, &dev_slots(c)->tokens, 0, B, c->h,
                                         c->bad_flag, st));
  int pending = 0;  // split-K partial sums of the last residual GEMM not yet in h
  for (int l = 0; l < d.L; ++l) {
    const LayerW &w = c->layers[l];
    const q2::QkvEpi e = qkv_epi(c, l, dpos, dseq);
    if (B <= kGemvRows) {
      TIMED(QWEN2_OP_QKV, q2::gemv_qkv(d, w, c->h, B, e, eps, c->normed, st,
                                       l == 0 && emb_fused ? &emb : nullptr));
    } else if (pending == 0 && q2::qkv_fuses_norm(d, B, c->splitk)) {
      TIMED(QWEN2_OP_QKV, q2::gemm_qkv_normed(d, w, c->h, d.H, B, eps, e, st));
    } else {
      TIMED(QWEN2_OP_NORM, q2::rmsnorm_rows_f16(c->h, d.H, w.attn_norm, d.H, B, eps, c->x16, d.H,
                                                nullptr, c->splitk.buf, pending, st));
      TIMED(QWEN2_OP_QKV, q2::gemm_qkv(d, w, c->x16, d.H, B, e, c->splitk, st));
    }
    pending = rows_rest(c, l, B, n_chunks, rows, seq1, st);
  }
  rows_head(c, B, rows, pending, st);
}

// Debug checks (QWEN2_DEBUG_CHECKS=1).  debug_begin marks the (sequence,
// position) slots a call may write and hashes every other cache word;
// debug_end hashes them again, scans the K / V the call wrote, its read-out
// hidden rows and its logits (when given) for non-finite values, waits for
// the stream, and returns QWEN2_E_DEBUG with the first offending value.
q2::DebugKv debug_args(qwen2_ctx *c) {
  const Dims &d = c->d;
  return q2::DebugKv{c->dbg_mask, d.hd, d.n_ctx, c->ldp, d.nkv, d.n_seq};
}

void debug_scan_kv(qwen2_ctx *c, unsigned long long *hash, unsigned long long *bk,
                   unsigned long long *bv, hipStream_t st) {
  const Dims &d = c->d;
  const size_t e16 = (size_t)d.L * d.n_seq * d.nkv * c->ldp * d.hd;
  q2::debug_kv(debug_args(c), c->kc, c->vc, c->kc16, c->vc16t, c->kv_elems, e16 / 2, hash, bk, bv,
               st);
}

int debug_begin(qwen2_ctx *c, const std::vector<std::pair<int, int>> &slots, hipStream_t st) {
  HIP_TRY(c, hipStreamSynchronize(st));  // (the previous check's kernels read the mask)
  std::fill(c->dbg_host.begin(), c->dbg_host.end(), 0);
  for (const auto &sp : slots) c->dbg_host[(size_t)sp.first * c->d.n_ctx + sp.second] = 1;
  HIP_TRY(c, hipMemcpy(c->dbg_mask, c->dbg_host.data(), c->dbg_host.size(), hipMemcpyHostToDevice));
  const unsigned long long init[8] = {0, 0, ~0ull, ~0ull, ~0ull, ~0ull, ~0ull, ~0ull};
  HIP_TRY(c, hipMemcpy(c->dbg, init, sizeof(init), hipMemcpyHostToDevice));
  debug_scan_kv(c, c->dbg + 0, c->dbg + 6, c->dbg + 7, st);
  HIP_TRY(c, hipGetLastError());
  return QWEN2_OK;
}

int debug_end(qwen2_ctx *c, const float *logits, int logit_rows, hipStream_t st) {
  const Dims &d = c->d;
  debug_scan_kv(c, c->dbg + 1, c->dbg + 2, c->dbg + 3, st);
  if (logits) q2::debug_nonfinite(logits, (size_t)logit_rows * d.V, c->dbg + 4, st);
  if (c->last_h) q2::debug_nonfinite(c->last_h, (size_t)c->last_rows * d.H, c->dbg + 5, st);
  HIP_TRY(c, hipGetLastError());
  HIP_TRY(c, hipStreamSynchronize(st));
  unsigned long long r[8];
  HIP_TRY(c, hipMemcpy(r, c->dbg, sizeof(r), hipMemcpyDeviceToHost));
  auto value = [&](const float *base, unsigned long long i, float *v) -> int {
    HIP_TRY(c, hipMemcpy(v, base + i, 4, hipMemcpyDeviceToHost));
    return QWEN2_OK;
  };
  char buf[256];
  if (r[0] != r[1])
    return set_err(c, QWEN2_E_DEBUG, "debug check: the KV cache changed outside this call's slots");
  for (int kv = 0; kv < 2; ++kv) {
    const unsigned long long w = r[2 + kv];
    if (w == ~0ull) continue;
    float v = 0.f;
    if (value(kv ? c->vc : c->kc, w, &v)) return QWEN2_E_HIP;
    const unsigned long long slot = w / d.hd;
    const int dim = (int)(w % d.hd), pos = (int)(slot % d.n_ctx);
    const int g = (int)((slot / d.n_ctx) % d.nkv), sq = (int)((slot / ((size_t)d.n_ctx * d.nkv)) % d.n_seq);
    const int l = (int)(slot / ((size_t)d.n_ctx * d.nkv * d.n_seq));
    snprintf(buf, sizeof(buf), "debug check: non-finite %s at layer %d, sequence %d, KV head %d, "
             "position %d, dim %d: %g", kv ? "V" : "K", l, sq, g, pos, dim, (double)v);
    return set_err(c, QWEN2_E_DEBUG, buf);
  }
  if (r[4] != ~0ull) {
    float v = 0.f;
    if (value(logits, r[4], &v)) return QWEN2_E_HIP;
    snprintf(buf, sizeof(buf), "debug check: non-finite logit at row %d, id %d: %g",
             (int)(r[4] / d.V), (int)(r[4] % d.V), (double)v);
    return set_err(c, QWEN2_E_DEBUG, buf);
  }
  if (r[5] != ~0ull) {
    float v = 0.f;
    if (value(c->last_h, r[5], &v)) return QWEN2_E_HIP;
    snprintf(buf, sizeof(buf), "debug check: non-finite hidden state at read-out row %d, dim %d: %g",
             (int)(r[5] / d.H), (int)(r[5] % d.H), (double)v);
    return set_err(c, QWEN2_E_DEBUG, buf);
  }
  return QWEN2_OK;
}

}  // namespace

extern "C" {

int qwen2_prefill(qwen2_ctx *c, int32_t seq, const int32_t *tokens, const int32_t *positions,
                  int32_t n, float *logits_dev, int32_t *argmax_dev, void *stream) {
  if (!c) return QWEN2_E_ARG;
  std::string msg;
  int rc = q2::check_prefill(&c->hp, seq, tokens, positions, n, &msg);
  if (rc) return set_err(c, rc, msg);
  hipStream_t st = (hipStream_t)stream;
  if (c->debug) {
    std::vector<std::pair<int, int>> ds;
    for (int i = 0; i < n; ++i) ds.emplace_back(seq, positions[i]);
    if ((rc = debug_begin(c, ds, st))) return rc;
  }
  std::vector<int32_t> seqs(n, seq);
  const int32_t *fields[3] = {tokens, positions, seqs.data()};
  int *df[3];
  const CallSlots slots{(const int *)(c->io + kSlotBytes), logits_dev, argmax_dev};
  rc = stage_call(c, st, slots, n, 3, fields, df);
  if (rc) return rc;
  for (int off = 0; off < n; off += c->max_rows) {
    const int M = std::min(c->max_rows, n - off);
    prefill_pass(c, M, off, df[1] + off, df[2] + off, {Seg{0, M, seq}}, positions + off, st);
    if (off + M == n) tail_row(c, M - 1, df[1] + off, df[2] + off, positions[n - 1], seq, st);
  }
  HIP_TRY(c, hipGetLastError());
  return c->debug ? debug_end(c, logits_dev, 1, st) : QWEN2_OK;
}

int qwen2_prefill_batch(qwen2_ctx *c, int32_t nb, const int32_t *seq_ids, const int32_t *lens,
                        const int32_t *tokens, const int32_t *positions, float *logits_dev,
                        int32_t *argmax_dev, void *stream) {
  if (!c) return QWEN2_E_ARG;
  std::string msg;
  int rc = q2::check_prefill_batch(&c->hp, nb, seq_ids, lens, tokens, positions, &msg);
  if (rc) return set_err(c, rc, msg);
  hipStream_t st = (hipStream_t)stream;
  const Dims &d = c->d;
  const int nhd = d.nh * d.hd;
  std::vector<int> end(nb);  // one past each sequence's last row
  int total = 0;
  for (int b = 0; b < nb; ++b) end[b] = total += lens[b];
  if (c->debug) {
    std::vector<std::pair<int, int>> ds;
    for (int b = 0, r = 0; b < nb; ++b)
      for (; r < end[b]; ++r) ds.emplace_back(seq_ids[b], positions[r]);
    if ((rc = debug_begin(c, ds, st))) return rc;
  }
  // Passes of up to max_rows consecutive rows; a sequence may straddle two.
  // At the end of each pass the residual rows and queries of the sequences
  // whose last row it holds are set aside (normed, o32: row b for sequence
  // b), and one read-out of all nb rows follows the last pass.
  std::vector<int32_t> f_tok, f_pos, f_seq;
  int b = 0;
  for (int off = 0; off < total; off += c->max_rows) {
    const int M = std::min(c->max_rows, total - off);
    std::vector<Seg> segs;
    std::vector<int32_t> src, dst;
    for (int r = off; r < off + M;) {
      while (end[b] <= r) ++b;
      const int stop = std::min(end[b], off + M);
      segs.push_back(Seg{r - off, stop - r, seq_ids[b]});
      if (stop == end[b]) {
        src.push_back(stop - 1 - off);
        dst.push_back(b);
      }
      r = stop;
    }
    const int k = (int)src.size();
    f_tok.assign(tokens + off, tokens + off + M);
    f_pos.assign(positions + off, positions + off + M);
    f_seq.clear();
    for (const Seg &g : segs) f_seq.insert(f_seq.end(), g.n, g.seq);
    f_tok.insert(f_tok.end(), src.begin(), src.end());
    f_pos.insert(f_pos.end(), dst.begin(), dst.end());
    f_seq.resize(M + k, 0);
    const int32_t *fields[3] = {f_tok.data(), f_pos.data(), f_seq.data()};
    int *df[3];
    const CallSlots slots{(const int *)(c->io + kSlotBytes), nullptr, nullptr};
    rc = stage_call(c, st, slots, M + k, 3, fields, df);
    if (rc) return rc;
    prefill_pass(c, M, 0, df[1], df[2], segs, positions + off, st);
    q2::copy_rows(c->h, d.H, df[0] + M, c->normed, d.H, df[1] + M, k, d.H, st);
    q2::copy_rows(c->q32, nhd, df[0] + M, c->o32, nhd, df[1] + M, k, nhd, st);
  }
  // read-out: the last layer from attention on, for the last row of each sequence
  std::vector<int32_t> t_pos(nb), t_seq(seq_ids, seq_ids + nb);
  for (int i = 0; i < nb; ++i) t_pos[i] = positions[end[i] - 1];
  const int32_t *fields[2] = {t_pos.data(), t_seq.data()};
  int *df[2];
  const CallSlots slots{nullptr, logits_dev, argmax_dev};
  rc = stage_call(c, st, slots, nb, 2, fields, df);
  if (rc) return rc;
  HIP_TRY(c, hipMemcpyAsync(c->h, c->normed, (size_t)nb * d.H * 4, hipMemcpyDeviceToDevice, st));
  HIP_TRY(c, hipMemcpyAsync(c->q32, c->o32, (size_t)nb * nhd * 4, hipMemcpyDeviceToDevice, st));
  const int n_chunks = chunks_for(*std::max_element(t_pos.begin(), t_pos.end()));
  const q2::RowInfo tail{df[0], df[1]};
  const int pending = rows_rest(c, d.L - 1, nb, n_chunks, tail, nb == 1 ? seq_ids[0] : -1, st);
  rows_head(c, nb, tail, pending, st);
  c->last_h = c->h;
  c->last_rows = nb;
  HIP_TRY(c, hipGetLastError());
  return c->debug ? debug_end(c, logits_dev, nb, st) : QWEN2_OK;
}

int qwen2_decode(qwen2_ctx *c, int32_t B, const int32_t *seq_ids, const int32_t *tokens_dev,
                 const int32_t *positions, float *logits_dev, int32_t *argmax_dev, void *stream) {
  if (!c) return QWEN2_E_ARG;
  std::string msg;
  int rc = q2::check_decode(&c->hp, B, seq_ids, positions, &msg);
  if (rc) return set_err(c, rc, msg);
  if (!tokens_dev) return set_err(c, QWEN2_E_ARG, "null tokens_dev");
  hipStream_t st = (hipStream_t)stream;
  if (c->debug) {
    std::vector<std::pair<int, int>> ds;
    for (int b = 0; b < B; ++b) ds.emplace_back(seq_ids[b], positions[b]);
    if ((rc = debug_begin(c, ds, st))) return rc;
  }
  const int32_t *fields[2] = {positions, seq_ids};
  int *df[2];
  const CallSlots slots{tokens_dev, logits_dev, argmax_dev};
  rc = stage_call(c, st, slots, B, 2, fields, df);
  if (rc) return rc;
  const int n_chunks = chunks_for(*std::max_element(positions, positions + B));
  const int seq1 = B == 1 ? seq_ids[0] : -1;  // a one-row step addresses its slot directly
  c->last_h = c->h;
  c->last_rows = B;
  if (!c->use_graphs || c->prof_mask) {
    decode_launches(c, B, n_chunks, df[0], df[1], seq1, st);
    HIP_TRY(c, hipGetLastError());
    return c->debug ? debug_end(c, logits_dev, B, st) : QWEN2_OK;
  }
  // What the captured launches depend on: the row count; the chunk count
  // (the chunked attention's grid, the one-row fused attention's key bound),
  // except for the fused attention of 2..8 rows, which reads it on the
  // device; the slot, for the one-row fused attention only.
  const bool fused = B <= kGemvRows && n_chunks * q2::kChunkKeys <= q2::kFusedKeys;
  const GraphKey key{(int)B, fused && B > 1 ? 0 : n_chunks, fused && B == 1 ? seq1 : -1};
  auto it = std::find_if(c->graphs.begin(), c->graphs.end(),
                         [&](const std::pair<GraphKey, hipGraphExec_t> &g) { return g.first == key; });
  if (it == c->graphs.end()) {
    hipGraph_t g = nullptr;
    hipGraphExec_t ge = nullptr;
    // capture on the library's own stream (the caller's may be the null
    // stream, which cannot be captured); the graph then runs on the caller's
    hipStream_t cs = c->cap_stream;
    HIP_TRY(c, hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal));
    decode_launches(c, B, n_chunks, df[0], df[1], seq1, cs);
    hipError_t e1 = hipStreamEndCapture(cs, &g);
    if (e1 != hipSuccess) return set_err(c, QWEN2_E_HIP, std::string("graph capture: ") + hipGetErrorString(e1));
    hipError_t e2 = hipGraphInstantiate(&ge, g, nullptr, nullptr, 0);
    (void)hipGraphDestroy(g);
    if (e2 != hipSuccess) return set_err(c, QWEN2_E_HIP, std::string("graph instantiate: ") + hipGetErrorString(e2));
    if (c->graphs.size() >= kMaxGraphs) {
      // the least recently used graph goes, once no replay of it can still
      // be in flight on this stream
      HIP_TRY(c, hipStreamSynchronize(st));
      (void)hipGraphExecDestroy(c->graphs.back().second);
      c->graphs.pop_back();
    }
    c->graphs.emplace_front(key, ge);
  } else if (it != c->graphs.begin()) {
    c->graphs.splice(c->graphs.begin(), c->graphs, it);
  }
  HIP_TRY(c, hipGraphLaunch(c->graphs.front().second, st));
  return c->debug ? debug_end(c, logits_dev, B, st) : QWEN2_OK;
}

int qwen2_next_token_probs(qwen2_ctx *c, const float *logits_dev, int32_t rows, float *probs_dev,
                           void *stream) {
  if (!c) return QWEN2_E_ARG;
  if (!logits_dev || !probs_dev) return set_err(c, QWEN2_E_ARG, "null logits or probs");
  if (rows < 1 || rows > c->dec_rows)
    return set_err(c, QWEN2_E_ARG, "rows must be in [1, max(n_seq, 8)]");
  hipStream_t st = (hipStream_t)stream;
  q2::softmax_rows(logits_dev, rows, c->d.V, c->prob_part, probs_dev, st);
  HIP_TRY(c, hipGetLastError());
  return QWEN2_OK;
}

int qwen2_set_stop_ids(qwen2_ctx *c, const int32_t *ids, int32_t n) {
  if (!c) return QWEN2_E_ARG;
  if (n < 0 || n > q2::kMaxStopIds || (n > 0 && !ids))
    return set_err(c, QWEN2_E_ARG, "between 0 and 8 stop ids");
  int32_t t[1 + q2::kMaxStopIds] = {n};
  for (int i = 0; i < n; ++i) {
    if (ids[i] < 0 || ids[i] >= c->d.V) return set_err(c, QWEN2_E_TOKEN, "stop id outside [0, n_vocab)");
    t[1 + i] = ids[i];
  }
  HIP_TRY(c, hipMemcpy(c->stop_ids, t, sizeof t, hipMemcpyHostToDevice));
  return QWEN2_OK;
}

int qwen2_read_stops(qwen2_ctx *c, int32_t *out_dev, int32_t clear, void *stream) {
  if (!c) return QWEN2_E_ARG;
  if (!out_dev) return set_err(c, QWEN2_E_ARG, "null out_dev");
  q2::read_stops(c->stop_pos, c->d.n_seq, out_dev, clear != 0, (hipStream_t)stream);
  HIP_TRY(c, hipGetLastError());
  return QWEN2_OK;
}

int qwen2_read_hidden(qwen2_ctx *c, int32_t which, float *out_dev, void *stream) {
  if (!c || !out_dev || (which != 0 && which != 1)) return set_err(c, QWEN2_E_ARG, "bad argument");
  if (!c->last_rows) return set_err(c, QWEN2_E_ARG, "no prefill or decode has run yet");
  const float *src = which == 0 ? c->last_h : c->normed;
  HIP_TRY(c, hipMemcpyAsync(out_dev, src, (size_t)c->last_rows * c->d.H * 4,
                            hipMemcpyDeviceToDevice, (hipStream_t)stream));
  return QWEN2_OK;
}

static int kv_copy(qwen2_ctx *c, int32_t layer, int32_t seq, int32_t pos0, int32_t n, float *k,
                   float *v, void *stream, bool to_cache) {
  if (!c || !k || !v || n <= 0 || layer < 0 || layer >= c->d.L)
    return set_err(c, QWEN2_E_ARG, "bad kv copy argument");
  if (seq < 0 || seq >= c->d.n_seq) return set_err(c, QWEN2_E_SEQ, "bad sequence slot");
  if (pos0 < 0 || (long long)pos0 + n > c->d.n_ctx)
    return set_err(c, QWEN2_E_POS, "kv range outside [0, n_ctx)");
  const q2::KVCache kv = kv_of(c);
  const size_t bytes = (size_t)n * c->d.hd * 4;
  const bool il = c->hp.rope_style == 1;  // K held in rotation-pair order (see pack_qkv)
  for (int g = 0; g < c->d.nkv; ++g) {
    float *ck = c->kc + kv.off(c->d, layer, seq, g, pos0);
    float *cv = c->vc + kv.off(c->d, layer, seq, g, pos0);
    float *bk = k + (size_t)g * n * c->d.hd, *bv = v + (size_t)g * n * c->d.hd;
    hipStream_t st = (hipStream_t)stream;
    if (to_cache) {
      if (il) q2::pair_order(bk, ck, n, c->d.hd, true, st);
      else HIP_TRY(c, hipMemcpyAsync(ck, bk, bytes, hipMemcpyDeviceToDevice, st));
      HIP_TRY(c, hipMemcpyAsync(cv, bv, bytes, hipMemcpyDeviceToDevice, st));
    } else {
      if (il) q2::pair_order(ck, bk, n, c->d.hd, false, st);
      else HIP_TRY(c, hipMemcpyAsync(bk, ck, bytes, hipMemcpyDeviceToDevice, st));
      HIP_TRY(c, hipMemcpyAsync(bv, cv, bytes, hipMemcpyDeviceToDevice, st));
    }
  }
  if (to_cache) {
    q2::kv_mirror(c->d, kv, layer, seq, pos0, n, (hipStream_t)stream);
    HIP_TRY(c, hipGetLastError());
  }
  return QWEN2_OK;
}

int qwen2_kv_read(qwen2_ctx *c, int32_t layer, int32_t seq, int32_t pos0, int32_t n, float *k_dev,
                  float *v_dev, void *stream) {
  return kv_copy(c, layer, seq, pos0, n, k_dev, v_dev, stream, false);
}

int qwen2_kv_write(qwen2_ctx *c, int32_t layer, int32_t seq, int32_t pos0, int32_t n,
                   const float *k_dev, const float *v_dev, void *stream) {
  return kv_copy(c, layer, seq, pos0, n, (float *)k_dev, (float *)v_dev, stream, true);
}

int qwen2_sync_status(qwen2_ctx *c, void *stream) {
  if (!c) return QWEN2_E_ARG;
  HIP_TRY(c, hipStreamSynchronize((hipStream_t)stream));
  unsigned flag = 0;
  HIP_TRY(c, hipMemcpy(&flag, c->bad_flag, 4, hipMemcpyDeviceToHost));
  if (flag) {
    HIP_TRY(c, hipMemset(c->bad_flag, 0, 4));
    return set_err(c, QWEN2_E_TOKEN, "a device-side token id was outside [0, n_vocab)");
  }
  return QWEN2_OK;
}

int qwen2_info(const qwen2_ctx *c, qwen2_info_t *o) {
  if (!c || !o) return QWEN2_E_ARG;
  memset(o, 0, sizeof *o);
  o->weight_bytes_f16 = c->w_f16;
  o->weight_bytes_f32 = c->w_f32;
  o->weight_bytes_alloc = c->warena_bytes;
  o->kv_bytes_per_pos = (uint64_t)c->d.L * 2 * c->d.nkv * c->d.hd * 4;
  o->kv_bytes = (uint64_t)c->kv_elems * 2 * 4;
  o->scratch_bytes = c->sarena_bytes;
  o->n_ctx = c->d.n_ctx;
  o->n_seq = c->d.n_seq;
  o->max_rows = c->max_rows;
  return QWEN2_OK;
}

int qwen2_prof_enable(qwen2_ctx *c, uint32_t mask) {
  if (!c) return QWEN2_E_ARG;
  if (mask && c->prof_ev.empty()) {
    c->prof_ev.resize(2 * kProfMax);
    for (auto &e : c->prof_ev) HIP_TRY(c, hipEventCreate(&e));
  }
  c->prof_mask = mask;
  return QWEN2_OK;
}

int qwen2_prof_read(qwen2_ctx *c, int32_t op, int32_t *launches, double *total_ms) {
  if (!c || !launches || !total_ms || op < 0 || op >= QWEN2_OP_COUNT)
    return set_err(c, QWEN2_E_ARG, "bad prof_read argument");
  int n = 0;
  double ms = 0.0;
  std::vector<std::pair<int, int>> keep;
  for (const auto &r : c->prof_rec) {
    if (r.first != op) {
      keep.push_back(r);
      continue;
    }
    HIP_TRY(c, hipEventSynchronize(c->prof_ev[2 * r.second + 1]));
    float t = 0.f;
    HIP_TRY(c, hipEventElapsedTime(&t, c->prof_ev[2 * r.second], c->prof_ev[2 * r.second + 1]));
    ms += t;
    ++n;
  }
  c->prof_rec.swap(keep);
  if (c->prof_rec.empty()) c->prof_used = 0;
  *launches = n;
  *total_ms = ms;
  return QWEN2_OK;
}

int qwen2_prof_repeat(qwen2_ctx *c, int32_t op, int32_t rows, int32_t iters, void *stream) {
  if (!c || op != QWEN2_OP_GATEUP || rows < 1 || rows > kGemvRows || iters < 1)
    return set_err(c, QWEN2_E_ARG, "prof_repeat supports QWEN2_OP_GATEUP with 1..8 rows");
  hipStream_t st = (hipStream_t)stream;
  for (int i = 0; i < iters; ++i) {
    const LayerW &w = c->layers[i % c->d.L];
    q2::gemv_swiglu(c->d, w, c->h, rows, c->a32, c->d.I_pad, c->hp.rms_eps, c->normed, st);
  }
  HIP_TRY(c, hipGetLastError());
  return QWEN2_OK;
}

const char *qwen2_last_error(const qwen2_ctx *c) {
  return c ? c->err.c_str() : g_load_error.c_str();
}

void qwen2_free(qwen2_ctx *c) { release(c); }

}  // extern "C"
