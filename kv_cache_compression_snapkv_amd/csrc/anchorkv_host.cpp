// Host side of the C ABI: argument checks, the byte plan, the cache layout,
// workspace layouts and the reference host packer / unpacker.  No HIP calls
// here except through run_compress / run_decode.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <climits>
#include <cstring>
#include <vector>
#include <algorithm>

#include "anchorkv_internal.hpp"

namespace akv {

static thread_local char g_err[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int obs_splits(const anchorkv_plan_info& p) {
  int64_t heads = (int64_t)p.units * p.H;
  int64_t want = (2048 + heads - 1) / heads;
  int64_t cap = std::max<int64_t>(1, p.N / 1024);
  return (int)std::max<int64_t>(1, std::min(want, cap));
}

CompressWs compress_ws_layout(const anchorkv_plan_info& p) {
  CompressWs w{};
  const int64_t U = p.units, H = p.H, N = p.N, D = p.D, A = p.A;
  w.S1 = obs_splits(p);
  w.GQp = padded_queries(p);
  const int64_t GQp = w.GQp;
  int64_t off = 0;
  auto take = [&](int64_t bytes) { int64_t o = off; off = round_up(off + bytes, 256); return o; };
  w.score = take(4 * U * H * N);
  w.ml = take(8 * U * H * GQp);
  w.o = take(4 * U * H * GQp * D);
  w.util = take(4 * U * 2 * H * N);
  w.gam = take(4 * U * 2 * H * N);
  w.rn2 = take(4 * U * 2 * H * N);
  w.aidx = take(4 * U * 2 * H * N);
  w.ml_part = take(8 * U * H * w.S1 * GQp);
  w.o_part = take(4 * U * H * w.S1 * GQp * D);
  w.ohl = take(2 * U * H * 2 * GQp * D);
  w.oo = take(4 * U * H * GQp);
  w.anchor_of = take(4 * U * H * N);
  w.vn2 = take(4 * U * H * N);
  w.uflag = take(U * H * ((N + 31) / 32));
  w.anorm = take(8 * U * 2 * H * A);
  w.pooled = take(4 * U * H * N);
  w.sel_list = take(4 * U * 2 * std::max<int64_t>(1, sel_stride(p)));
  w.sel_aux = take(8 * U * 2 * std::max<int64_t>(1, sel_stride(p)));
  w.sel_groups = take(8 * U * 2 * ((H * N + 1023) / 1024) + 8 * U * 2);
  const bool cover = p.params.anchor_mode == ANCHORKV_ANCHORS_COVER;
  w.cover_mc = take(cover ? 4 * U * H * N : 0);
  w.cover_list = take(cover ? 4 * U * H * std::max<int64_t>(1, (int64_t)p.k_scored + p.k_uniform) : 0);
  w.rope_cs = take(p.params.rope ? 8 * N * (D / 2) : 0);
  w.total = off;
  return w;
}

DecodeWs decode_ws_layout(const anchorkv_plan_info& p) {
  DecodeWs w{};
  const int64_t U = p.units, H = p.H, G = p.G, D = p.D;
  w.S2 = p.decode_splits;
  int64_t off = 0;
  auto take = [&](int64_t bytes) { int64_t o = off; off = round_up(off + bytes, 256); return o; };
  w.part_ml = take(8 * U * H * w.S2 * G);
  w.part_acc = take(4 * U * H * w.S2 * G * D);
  // tail ranges: enough workgroups to cover the chip (about 2048) when the
  // tail is long, at most 16 per head
  w.St = (int)std::min<int64_t>(16, std::max<int64_t>(1, (2048 + U * H - 1) / (U * H)));
  w.tail_ml = take(8 * U * H * w.St * G);
  w.tail_acc = take(4 * U * H * w.St * G * D);
  w.total = off;
  return w;
}

// Token splits per (unit, head) of the decode pass.  One block per split
// walks its 1024-token chunks after reading the head's anchors twice (keys for
// the logit table, values for the output), and one or two blocks fit a
// compute unit.  Fewest rounds of resident blocks times bytes per block;
// fewer splits on ties (each split adds anchor reads and a partial to merge).
static int decode_split_count(const anchorkv_plan_info& p) {
  const int64_t heads = (int64_t)p.units * p.H;
  const int64_t C = p.n_chunks;   // splits start on 1024-token chunk boundaries
  const int64_t slots = 256 * (int64_t)decode_blocks_per_cu(p.G, p.A, p.dtype == ANCHORKV_F32, p.params.codec);
  const int64_t chunk_bytes = 8 * 1024 + rec_bytes_of(p) * (int64_t)records_per_unit(p) / std::max<int64_t>(1, p.H * C);
  const int64_t anchor_bytes = 2 * (int64_t)p.A * p.D * p.elem_bytes;
  int best = 1;
  int64_t best_cost = INT64_MAX;
  for (int64_t s = 1; s <= std::min<int64_t>(C, 64); ++s) {
    const int64_t per = (C + s - 1) / s;
    const int64_t cost = ((heads * s + slots - 1) / slots) * (per * chunk_bytes + anchor_bytes);
    if (cost < best_cost) { best_cost = cost; best = (int)s; }
  }
  return best;
}

static void layout(anchorkv_plan_info* p) {
  const int64_t H = p->H, N = p->N, D = p->D, A = p->A, e = p->elem_bytes, C = p->n_chunks;
  const int64_t RB = rec_bytes_of(*p);
  int64_t off = kHeaderBytes;
  p->off_anchor_k = off; off += H * A * D * e;
  p->off_anchor_v = off; off += H * A * D * e;
  if (p->joint) {
    // one section: key records first, then value records (the split is the data's)
    p->off_res_k = off;
    p->off_res_v = off;
    off += RB * p->R_total;
  } else {
    p->off_res_k = off; off += RB * p->R_K;
    p->off_res_v = off; off += RB * p->R_V;
  }
  p->off_words = off; off += 8 * H * N;
  p->off_chunk_k = off; off += 4 * H * C;
  p->off_chunk_v = off; off += 4 * H * C;
  p->off_positions = off; off += 4 * H * A;
  p->unit_bytes = off;
  p->unit_stride = round_up(off, 16);
  p->cache_bytes = p->unit_stride * p->units;
  p->decode_splits = decode_split_count(*p);
  p->compress_workspace_bytes = compress_ws_layout(*p).total;
  p->decode_workspace_bytes = decode_ws_layout(*p).total;
}

void fill_header(const anchorkv_plan_info& p, UnitHeader* h) {
  std::memset(h, 0, sizeof(*h));
  h->magic = kMagic;
  h->version = 1;
  h->H = p.H; h->G = p.G; h->N = p.N; h->D = p.D; h->n_obs = p.n_obs; h->dtype = p.dtype; h->window = p.window;
  h->theta = p.theta;
  h->A = p.A; h->k_scored = p.k_scored; h->k_uniform = p.k_uniform; h->R_K = p.R_K; h->R_V = p.R_V;
  h->n_chunks = p.n_chunks;
  h->off_anchor_k = p.off_anchor_k; h->off_anchor_v = p.off_anchor_v;
  h->off_res_k = p.off_res_k; h->off_res_v = p.off_res_v; h->off_words = p.off_words;
  h->off_chunk_k = p.off_chunk_k; h->off_chunk_v = p.off_chunk_v; h->off_positions = p.off_positions;
  h->unit_bytes = p.unit_bytes; h->unit_stride = p.unit_stride;
  h->anchor_div = p.params.anchor_div; h->pool = p.params.pool; h->group = p.params.group;
  h->pool_kv_jointly = p.params.pool_kv_jointly; h->rho = p.params.rho;
  h->R_total = p.R_total;
  h->codec = p.params.codec;
  for (int i = 0; i < 4; ++i) h->signs[i] = p.params.hadamard_signs[i];
  h->rope = p.params.rope;
  h->rope_theta = p.params.rope_theta;
}

// SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
// generators", 2014): advance the state by the golden-ratio increment, then
// mix it with two multiply-xorshift rounds.
static uint64_t splitmix64(uint64_t& state) {
  uint64_t z = (state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
static constexpr uint64_t kSignSeed = 0x416E63686F724B56ull;

static void params_default(anchorkv_params* q, float theta, int32_t window) {
  std::memset(q, 0, sizeof(*q));
  q->theta = theta;
  q->window = window;
  q->anchor_div = 128;
  q->rho = 0.7;
  q->pool = 7;
  q->group = kGroup;
  q->pool_kv_jointly = 0;
  q->codec = ANCHORKV_CODEC_AFFINE;
  q->anchor_mode = ANCHORKV_ANCHORS_UNIFORM;
  q->cover_rounds = 8;
  q->rope = 0;
  q->rope_theta = 500000.0f;
  uint64_t st = kSignSeed;
  const uint64_t a = splitmix64(st), b = splitmix64(st);
  q->hadamard_signs[0] = (uint32_t)a; q->hadamard_signs[1] = (uint32_t)(a >> 32);
  q->hadamard_signs[2] = (uint32_t)b; q->hadamard_signs[3] = (uint32_t)(b >> 32);
}

static int check_params(const anchorkv_params& q) {
  if (!(q.theta > 0.0f) || !(q.theta <= 1024.0f))
    return fail(ANCHORKV_E_ARG, "anchorkv_plan: theta must be in (0, 1024]");
  if (q.anchor_div < 1) return fail(ANCHORKV_E_ARG, "anchorkv_plan: anchor_div %d must be >= 1", q.anchor_div);
  if (!(q.rho >= 0.0 && q.rho <= 1.0)) return fail(ANCHORKV_E_ARG, "anchorkv_plan: rho must be in [0, 1]");
  if (q.pool < 1 || q.pool > kMaxPool || q.pool % 2 == 0)
    return fail(ANCHORKV_E_ARG, "anchorkv_plan: pool %d must be odd and in [1, %d]", q.pool, kMaxPool);
  if (q.group != kGroup) return fail(ANCHORKV_E_ARG, "anchorkv_plan: codec group %d: only %d is supported", q.group, kGroup);
  if (q.pool_kv_jointly != 0 && q.pool_kv_jointly != 1)
    return fail(ANCHORKV_E_ARG, "anchorkv_plan: pool_kv_jointly %d must be 0 or 1", q.pool_kv_jointly);
  if (q.codec != ANCHORKV_CODEC_AFFINE && q.codec != ANCHORKV_CODEC_HADAMARD_LM)
    return fail(ANCHORKV_E_ARG, "anchorkv_plan: codec %d is not 0 (affine) or 1 (Hadamard / Lloyd-Max)", q.codec);
  if (q.anchor_mode != ANCHORKV_ANCHORS_UNIFORM && q.anchor_mode != ANCHORKV_ANCHORS_COVER)
    return fail(ANCHORKV_E_ARG, "anchorkv_plan: anchor_mode %d is not 0 (uniform) or 1 (coverage)", q.anchor_mode);
  if (q.cover_rounds < 1 || q.cover_rounds > 1024)
    return fail(ANCHORKV_E_ARG, "anchorkv_plan: cover_rounds %d must be in [1, 1024]", q.cover_rounds);
  if (q.rope != 0 && q.rope != 1) return fail(ANCHORKV_E_ARG, "anchorkv_plan: rope %d must be 0 or 1", q.rope);
  if (!(q.rope_theta > 1.0f) || !(q.rope_theta <= 1e10f))
    return fail(ANCHORKV_E_ARG, "anchorkv_plan: rope_theta must be in (1, 1e10]");
  if (q.rope && q.codec != ANCHORKV_CODEC_AFFINE)
    return fail(ANCHORKV_E_ARG, "anchorkv_plan: pre-RoPE keys (rope = 1) need the group-affine codec");
  for (int i = 0; i < (int)(sizeof(q.reserved) / sizeof(q.reserved[0])); ++i)
    if (q.reserved[i] != 0) return fail(ANCHORKV_E_ARG, "anchorkv_plan: reserved parameter fields must be zero");
  return 0;
}

static int plan_impl(const anchorkv_dims* d, const anchorkv_params* prm, anchorkv_plan_info* out) {
  if (!d || !prm || !out) return fail(ANCHORKV_E_ARG, "anchorkv_plan: null argument");
  if (int rc = check_params(*prm)) return rc;
  const float theta = prm->theta;
  const int32_t window = prm->window;
  if (d->dtype != ANCHORKV_BF16 && d->dtype != ANCHORKV_F32)
    return fail(ANCHORKV_E_DTYPE, "anchorkv_plan: dtype %d is not bf16 (1) or f32 (2)", d->dtype);
  if (d->head_dim != kHeadDim) return fail(ANCHORKV_E_SHAPE, "anchorkv_plan: head_dim %d != 128", d->head_dim);
  if (d->units < 1 || d->kv_heads < 1 || d->q_per_kv < 1 || d->n_tokens < 1)
    return fail(ANCHORKV_E_SHAPE, "anchorkv_plan: units, kv_heads, q_per_kv, n_tokens must be >= 1");
  if (d->n_obs < 1 || d->n_obs > d->n_tokens)
    return fail(ANCHORKV_E_SHAPE, "anchorkv_plan: n_obs %d outside [1, n_tokens]", d->n_obs);
  if (window < 1 || window > d->n_tokens)
    return fail(ANCHORKV_E_SHAPE, "anchorkv_plan: window %d outside [1, n_tokens]", window);
  if ((int64_t)d->kv_heads * d->n_tokens > (1ll << 30) || (int64_t)d->q_per_kv * d->n_obs > 4096)
    return fail(ANCHORKV_E_SHAPE, "anchorkv_plan: kv_heads*n_tokens or q_per_kv*n_obs too large");

  anchorkv_plan_info p;
  std::memset(&p, 0, sizeof(p));
  p.params = *prm;
  p.units = d->units; p.H = d->kv_heads; p.G = d->q_per_kv; p.N = d->n_tokens; p.D = d->head_dim;
  p.n_obs = d->n_obs; p.dtype = d->dtype; p.elem_bytes = d->dtype == ANCHORKV_BF16 ? 2 : 4;
  p.window = window; p.theta = theta;
  const int64_t H = p.H, N = p.N, D = p.D, e = p.elem_bytes, W = window;
  const int64_t C = (N + kChunk - 1) / kChunk;
  p.n_chunks = (int32_t)C;
  const double th = (double)theta;
  // Per head and side: B = theta*N*D*e bytes; anchors cost D*e + 2 (their half of the int32
  // position), every token a 4-byte pointer, every chunk a 4-byte offset, the header 128/H.
  const double B = th * (double)(N * D * e);
  const double amax_d = std::floor((B - 4.0 * (double)N - 4.0 * (double)C - 128.0 / (double)H) / (double)(D * e + 2));
  if (amax_d < (double)W)
    return fail(ANCHORKV_E_BUDGET, "anchorkv_plan: theta %.6g cannot pay for %d window anchors and the pointers", th, window);
  const int64_t A_max = (int64_t)std::min(amax_d, (double)N);   // at most N anchors are ever usable
  const int64_t k_nw = std::max<int64_t>(0, std::min(std::min(N / prm->anchor_div, A_max - W), N - W));
  const int64_t k_s = std::min(k_nw, (int64_t)std::floor(prm->rho * (double)k_nw));
  const int64_t A = W + k_nw;
  if (A > kMaxAnchors) return fail(ANCHORKV_E_SHAPE, "anchorkv_plan: %lld anchors exceed the 15-bit index", (long long)A);
  p.A = (int32_t)A; p.k_scored = (int32_t)k_s; p.k_uniform = (int32_t)(k_nw - k_s);
  const int64_t budget = (int64_t)std::floor(th * (double)(H * N * D * e));
  const int64_t fixed = 128 + H * (A * D * e + 4 * N + 2 * A + 4 * C);
  const int64_t rec = rec_bytes_of(prm->codec);   // D/4 + D/8, or D/4 + 4 (D = 128)
  const int64_t R = std::max<int64_t>(0, std::min(H * (N - A), (budget - fixed) / rec));
  p.R_K = p.R_V = (int32_t)R;
  p.budget_bytes_per_side = budget;
  p.used_bytes_k = fixed + R * rec;
  p.used_bytes_v = fixed + R * rec;
  if (prm->pool_kv_jointly) {
    // both sides' remainders pooled: R_total = min(2H(N-A), floor(2(budget - fixed)/rec))
    const int64_t Rt = std::max<int64_t>(0, std::min(2 * H * (N - A), 2 * (budget - fixed) / rec));
    if (Rt > INT32_MAX) return fail(ANCHORKV_E_SHAPE, "anchorkv_plan: too many residual records");
    p.joint = 1;
    p.R_total = (int32_t)Rt;
    // the split between the sides is the data's: each side is charged half of the records here
    p.used_bytes_k = fixed + (Rt / 2) * rec;
    p.used_bytes_v = fixed + (Rt - Rt / 2) * rec;
  }
  layout(&p);
  p.compression_ratio = (double)(2 * H * N * D * e) / (double)p.unit_bytes;
  if (int rc = compress_supports(p)) return rc;
  if (int rc = decode_supports(p)) return rc;
  *out = p;
  return 0;
}

// Plan of `units` units from a host copy of a unit header.
static int plan_from_header_impl(const void* header_host, int32_t units, anchorkv_plan_info* out, const char* fn) {
  if (!header_host || !out || units < 1) return fail(ANCHORKV_E_ARG, "%s: bad argument", fn);
  UnitHeader h;
  std::memcpy(&h, header_host, sizeof(h));
  if (h.magic != kMagic || h.version != 1) return fail(ANCHORKV_E_LAYOUT, "%s: bad magic/version", fn);
  anchorkv_dims d{units, h.H, h.G, h.N, h.D, h.n_obs, h.dtype};
  anchorkv_params q;
  params_default(&q, h.theta, h.window);
  q.anchor_div = h.anchor_div; q.rho = h.rho; q.pool = h.pool; q.group = h.group;
  q.pool_kv_jointly = h.pool_kv_jointly;
  q.codec = h.codec;
  for (int i = 0; i < 4; ++i) q.hadamard_signs[i] = h.signs[i];
  q.rope = h.rope;
  q.rope_theta = h.rope_theta;
  int rc = plan_impl(&d, &q, out);
  if (rc) return rc == ANCHORKV_E_ARG ? fail(ANCHORKV_E_LAYOUT, "%s: header parameters are invalid", fn) : rc;
  if (out->A != h.A || out->R_K != h.R_K || out->R_V != h.R_V || out->R_total != h.R_total ||
      out->unit_bytes != h.unit_bytes ||
      out->off_words != h.off_words || out->k_scored != h.k_scored || out->unit_stride != h.unit_stride)
    return fail(ANCHORKV_E_LAYOUT, "%s: header does not match its own plan", fn);
  return 0;
}

}  // namespace akv

using namespace akv;

extern "C" {

const char* anchorkv_version(void) { return "anchorkv-mi355x 0.1 (gfx950)"; }

const char* anchorkv_last_error(void) { return g_err; }

void anchorkv_params_default(anchorkv_params* params, float theta, int32_t window) {
  if (params) params_default(params, theta, window);
}

int anchorkv_plan(const anchorkv_dims* dims, const anchorkv_params* params, anchorkv_plan_info* out) {
  return plan_impl(dims, params, out);
}

int anchorkv_plan_from_header(const void* header_host, int32_t units, anchorkv_plan_info* out) {
  return plan_from_header_impl(header_host, units, out, "anchorkv_plan_from_header");
}

int anchorkv_cache_layout(const void* header_host, anchorkv_layout* out) {
  if (!out) return fail(ANCHORKV_E_ARG, "anchorkv_cache_layout: null argument");
  anchorkv_plan_info p;
  if (int rc = plan_from_header_impl(header_host, 1, &p, "anchorkv_cache_layout")) return rc;
  std::memset(out, 0, sizeof(*out));
  out->off_anchor_k = p.off_anchor_k; out->off_anchor_v = p.off_anchor_v;
  out->off_res_k = p.off_res_k; out->off_res_v = p.off_res_v; out->off_words = p.off_words;
  out->off_chunk_k = p.off_chunk_k; out->off_chunk_v = p.off_chunk_v; out->off_positions = p.off_positions;
  out->unit_bytes = p.unit_bytes; out->unit_stride = p.unit_stride;
  out->A = p.A; out->R_K = p.R_K; out->R_V = p.R_V; out->n_chunks = p.n_chunks; out->record_bytes = rec_bytes_of(p);
  return 0;
}

int anchorkv_decode_workspace_bytes(const void* header_host, int32_t units, size_t* out) {
  if (!out) return fail(ANCHORKV_E_ARG, "anchorkv_decode_workspace_bytes: null argument");
  anchorkv_plan_info p;
  if (int rc = plan_from_header_impl(header_host, units, &p, "anchorkv_decode_workspace_bytes")) return rc;
  *out = (size_t)p.decode_workspace_bytes;
  return 0;
}

int anchorkv_workspace_offsets(const anchorkv_plan_info* plan, int64_t out[8]) {
  if (!plan || !out) return fail(ANCHORKV_E_ARG, "anchorkv_workspace_offsets: null argument");
  CompressWs w = compress_ws_layout(*plan);
  out[0] = w.score; out[1] = w.ml; out[2] = w.o; out[3] = w.util;
  out[4] = w.gam; out[5] = w.rn2; out[6] = w.aidx; out[7] = w.GQp;
  return 0;
}

int anchorkv_compress(const anchorkv_plan_info* plan, const void* K, const void* V, const void* Q_obs,
                      void* cache, size_t cache_bytes, void* workspace, size_t workspace_bytes, void* stream) {
  if (!plan || !K || !V || !Q_obs || !cache || !workspace) return fail(ANCHORKV_E_ARG, "anchorkv_compress: null argument");
  if ((int64_t)cache_bytes < plan->cache_bytes)
    return fail(ANCHORKV_E_SMALL_BUFFER, "anchorkv_compress: cache %zu < %lld bytes", cache_bytes, (long long)plan->cache_bytes);
  if ((int64_t)workspace_bytes < plan->compress_workspace_bytes)
    return fail(ANCHORKV_E_SMALL_BUFFER, "anchorkv_compress: workspace %zu < %lld bytes", workspace_bytes,
                (long long)plan->compress_workspace_bytes);
  if (((uintptr_t)K | (uintptr_t)V | (uintptr_t)Q_obs | (uintptr_t)cache | (uintptr_t)workspace) & 15)
    return fail(ANCHORKV_E_ARG, "anchorkv_compress: buffers must be 16-byte aligned");
  return run_compress(*plan, K, V, Q_obs, cache, workspace, stream);
}

int anchorkv_decode_attn(const anchorkv_plan_info* plan, const void* cache, size_t cache_bytes, const void* q, float* o,
                         void* workspace, size_t workspace_bytes, void* stream) {
  if (!plan || !cache || !q || !o || !workspace) return fail(ANCHORKV_E_ARG, "anchorkv_decode_attn: null argument");
  if ((int64_t)cache_bytes < plan->cache_bytes)
    return fail(ANCHORKV_E_SMALL_BUFFER, "anchorkv_decode_attn: cache %zu < %lld bytes", cache_bytes,
                (long long)plan->cache_bytes);
  if ((int64_t)workspace_bytes < plan->decode_workspace_bytes)
    return fail(ANCHORKV_E_SMALL_BUFFER, "anchorkv_decode_attn: workspace %zu < %lld bytes", workspace_bytes,
                (long long)plan->decode_workspace_bytes);
  if (((uintptr_t)cache | (uintptr_t)q | (uintptr_t)o | (uintptr_t)workspace) & 15)
    return fail(ANCHORKV_E_ARG, "anchorkv_decode_attn: buffers must be 16-byte aligned");
  return run_decode(*plan, cache, q, o, workspace, stream);
}

int anchorkv_decode_attn_noalloc(const anchorkv_plan_info* plan, const void* cache, size_t cache_bytes, const void* q,
                                 float* o, void* stream) {
  if (!plan || !cache || !q || !o) return fail(ANCHORKV_E_ARG, "anchorkv_decode_attn_noalloc: null argument");
  if ((int64_t)cache_bytes < plan->cache_bytes)
    return fail(ANCHORKV_E_SMALL_BUFFER, "anchorkv_decode_attn_noalloc: cache %zu < %lld bytes", cache_bytes,
                (long long)plan->cache_bytes);
  if (((uintptr_t)cache | (uintptr_t)q | (uintptr_t)o) & 15)
    return fail(ANCHORKV_E_ARG, "anchorkv_decode_attn_noalloc: buffers must be 16-byte aligned");
  return run_decode_noalloc(*plan, cache, q, o, stream);
}

int anchorkv_decode_attn_tail(const anchorkv_plan_info* plan, const void* cache, size_t cache_bytes, const void* q,
                              const void* K_tail, const void* V_tail, int32_t n_tail, int32_t tail_cap, float* o,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (!plan || !cache || !q || !o || !workspace) return fail(ANCHORKV_E_ARG, "anchorkv_decode_attn_tail: null argument");
  if ((int64_t)cache_bytes < plan->cache_bytes)
    return fail(ANCHORKV_E_SMALL_BUFFER, "anchorkv_decode_attn_tail: cache %zu < %lld bytes", cache_bytes,
                (long long)plan->cache_bytes);
  if (n_tail < 0 || tail_cap < n_tail)
    return fail(ANCHORKV_E_ARG, "anchorkv_decode_attn_tail: need 0 <= n_tail (%d) <= tail_cap (%d)", n_tail, tail_cap);
  if (n_tail > 0 && (!K_tail || !V_tail)) return fail(ANCHORKV_E_ARG, "anchorkv_decode_attn_tail: null tail");
  if ((int64_t)workspace_bytes < plan->decode_workspace_bytes)
    return fail(ANCHORKV_E_SMALL_BUFFER, "anchorkv_decode_attn_tail: workspace %zu < %lld bytes", workspace_bytes,
                (long long)plan->decode_workspace_bytes);
  if (((uintptr_t)cache | (uintptr_t)q | (uintptr_t)o | (uintptr_t)workspace | (uintptr_t)K_tail | (uintptr_t)V_tail) & 15)
    return fail(ANCHORKV_E_ARG, "anchorkv_decode_attn_tail: buffers must be 16-byte aligned");
  return run_decode_tail(*plan, cache, q, K_tail, V_tail, n_tail, tail_cap, o, workspace, stream);
}

// ---------------------------------------------------------------- host packer
// Code word j of a record holds coordinates j + 16c (c = 0..7) in bits 2c..2c+1.
int anchorkv_unit_pack_host(const anchorkv_plan_info* p, const anchorkv_unit_arrays* in, void* unit_out) {
  if (!p || !in || !unit_out || !in->positions || !in->anchors_k || !in->anchors_v || !in->idx || !in->gamma16 ||
      !in->flag || !in->codes || !in->scale16 || !in->zero16)
    return fail(ANCHORKV_E_ARG, "anchorkv_unit_pack_host: null argument");
  const int64_t H = p->H, N = p->N, D = p->D, A = p->A, e = p->elem_bytes, C = p->n_chunks;
  uint8_t* base = (uint8_t*)unit_out;
  std::memset(base, 0, (size_t)p->unit_bytes);
  UnitHeader hd;
  fill_header(*p, &hd);
  std::memcpy(base, &hd, sizeof(hd));
  std::memcpy(base + p->off_anchor_k, in->anchors_k, (size_t)(H * A * D * e));
  std::memcpy(base + p->off_anchor_v, in->anchors_v, (size_t)(H * A * D * e));
  std::memcpy(base + p->off_positions, in->positions, (size_t)(4 * H * A));
  uint32_t* words = (uint32_t*)(base + p->off_words);
  const int64_t RB = rec_bytes_of(*p);
  const bool hlm = p->params.codec == ANCHORKV_CODEC_HADAMARD_LM;
  int64_t r = 0;   // record index from the section start (joint: runs on from the key records)
  for (int s = 0; s < 2; ++s) {
    uint8_t* rec = base + (s ? p->off_res_v : p->off_res_k);
    int32_t* chunk = (int32_t*)(base + (s ? p->off_chunk_v : p->off_chunk_k));
    if (!p->joint) r = 0;
    const int64_t r0 = r;
    const int64_t cap = p->joint ? p->R_total : (s ? p->R_V : p->R_K);
    for (int64_t h = 0; h < H; ++h) {
      for (int64_t t = 0; t < N; ++t) {
        const int64_t i = (s * H + h) * N + t;
        if (t % kChunk == 0) chunk[h * C + t / kChunk] = (int32_t)r;
        const int32_t a = in->idx[i];
        if (a < 0 || a >= A) return fail(ANCHORKV_E_LAYOUT, "pack: anchor index %d out of range", a);
        uint32_t w = (uint32_t)a | ((uint32_t)in->gamma16[i] << 16);
        if (in->flag[i]) {
          if (r >= cap) return fail(ANCHORKV_E_LAYOUT, "pack: more flagged tokens than %lld records", (long long)cap);
          w |= 0x8000u;
          uint16_t cw[16] = {0};
          const uint8_t* cd = in->codes + i * D;
          for (int d = 0; d < D; ++d) cw[d % 16] |= (uint16_t)((cd[d] & 3u) << (2 * (d / 16)));
          uint8_t* out = rec + r * RB;
          std::memcpy(out, cw, 32);
          if (hlm) {
            const uint16_t sg[2] = {in->scale16[i * (D / kGroup)], 0};
            std::memcpy(out + 32, sg, 4);
          } else {
            for (int g = 0; g < D / kGroup; ++g) {
              uint16_t sz[2] = {in->scale16[i * (D / kGroup) + g], in->zero16[i * (D / kGroup) + g]};
              std::memcpy(out + 32 + 4 * g, sz, 4);
            }
          }
          ++r;
        }
        words[(h * N + t) * 2 + s] = w;
      }
    }
    if (!p->joint && r - r0 != cap)
      return fail(ANCHORKV_E_LAYOUT, "pack: %lld flagged tokens on side %d, plan has %lld", (long long)(r - r0), s,
                  (long long)cap);
  }
  if (p->joint && r != p->R_total)
    return fail(ANCHORKV_E_LAYOUT, "pack: %lld flagged token-sides, plan has %lld", (long long)r, (long long)p->R_total);
  return 0;
}

int anchorkv_unit_unpack_host(const anchorkv_plan_info* p, const void* unit_in, anchorkv_unit_arrays* out) {
  if (!p || !unit_in || !out) return fail(ANCHORKV_E_ARG, "anchorkv_unit_unpack_host: null argument");
  const int64_t H = p->H, N = p->N, D = p->D, A = p->A, e = p->elem_bytes, C = p->n_chunks;
  const uint8_t* base = (const uint8_t*)unit_in;
  UnitHeader hd;
  std::memcpy(&hd, base, sizeof(hd));
  if (hd.magic != kMagic || hd.A != p->A || hd.N != p->N || hd.H != p->H || hd.R_K != p->R_K || hd.R_V != p->R_V ||
      hd.R_total != p->R_total)
    return fail(ANCHORKV_E_LAYOUT, "unpack: header does not match the plan");
  if (out->anchors_k) std::memcpy(out->anchors_k, base + p->off_anchor_k, (size_t)(H * A * D * e));
  if (out->anchors_v) std::memcpy(out->anchors_v, base + p->off_anchor_v, (size_t)(H * A * D * e));
  if (out->positions) std::memcpy(out->positions, base + p->off_positions, (size_t)(4 * H * A));
  const uint32_t* words = (const uint32_t*)(base + p->off_words);
  const int64_t RB = rec_bytes_of(*p);
  const bool hlm = p->params.codec == ANCHORKV_CODEC_HADAMARD_LM;
  int64_t r = 0;   // record index from the section start (joint: runs on from the key records)
  for (int s = 0; s < 2; ++s) {
    const uint8_t* rec = base + (s ? p->off_res_v : p->off_res_k);
    const int32_t* chunk = (const int32_t*)(base + (s ? p->off_chunk_v : p->off_chunk_k));
    if (!p->joint) r = 0;
    const int64_t r0 = r;
    const int64_t cap = p->joint ? p->R_total : (s ? p->R_V : p->R_K);
    for (int64_t h = 0; h < H; ++h) {
      for (int64_t t = 0; t < N; ++t) {
        const int64_t i = (s * H + h) * N + t;
        if (t % kChunk == 0 && chunk[h * C + t / kChunk] != r)
          return fail(ANCHORKV_E_LAYOUT, "unpack: chunk offset mismatch at side %d head %lld chunk %lld", s,
                      (long long)h, (long long)(t / kChunk));
        const uint32_t w = words[(h * N + t) * 2 + s];
        if (out->idx) out->idx[i] = (int32_t)(w & 0x7FFFu);
        if (out->gamma16) out->gamma16[i] = (uint16_t)(w >> 16);
        const bool f = (w & 0x8000u) != 0;
        if (out->flag) out->flag[i] = f ? 1 : 0;
        if (f) {
          if (r >= cap) return fail(ANCHORKV_E_LAYOUT, "unpack: more flags than records on side %d", s);
          const uint8_t* in = rec + r * RB;
          uint16_t cw[16];
          std::memcpy(cw, in, 32);
          if (out->codes)
            for (int d = 0; d < D; ++d) out->codes[i * D + d] = (uint8_t)((cw[d % 16] >> (2 * (d / 16))) & 3u);
          for (int g = 0; g < D / kGroup; ++g) {
            uint16_t sz[2];
            if (hlm) {
              std::memcpy(sz, in + 32, 4);
              if (g > 0) sz[0] = 0;
              sz[1] = 0;
            } else {
              std::memcpy(sz, in + 32 + 4 * g, 4);
            }
            if (out->scale16) out->scale16[i * (D / kGroup) + g] = sz[0];
            if (out->zero16) out->zero16[i * (D / kGroup) + g] = sz[1];
          }
          ++r;
        }
      }
    }
    if (!p->joint && r - r0 != cap)
      return fail(ANCHORKV_E_LAYOUT, "unpack: %lld flags on side %d, plan has %lld", (long long)(r - r0), s,
                  (long long)cap);
  }
  if (p->joint && r != p->R_total)
    return fail(ANCHORKV_E_LAYOUT, "unpack: %lld flagged token-sides, plan has %lld", (long long)r,
                (long long)p->R_total);
  return 0;
}

}  // extern "C"
