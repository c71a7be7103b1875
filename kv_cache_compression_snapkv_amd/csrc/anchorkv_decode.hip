// Decode attention over the compressed cache (gfx950).
//
// For q-head g of KV head h (Pith review of AnchorKV, "What carries the
// argument": x^_t = gamma_t x_a(t) + r~_t):
//   logit_t = gamma^K_t <q, k_a> / sqrt(D) + [t in R_K] <q, r~^K_t> / sqrt(D)
//   o = sum_t p_t (gamma^V_t v_a(t) + [t in R_V] r~^V_t) / sum_t p_t
// computed without reconstructing K or V: the anchor logits <q, k_a> form a
// per-head table S[g][a]; the value side scatters p_t gamma^V_t into
// w[g][a(t)] and finishes with o = (w V_anchors + sum p r~^V) / l.  The
// token stream is split into 1024-token-aligned ranges per (unit, head);
// each range keeps its own online-softmax state and a combine kernel merges
// them.  Exponentials are base 2 with log2(e)/sqrt(D) folded into S.
#include "device_common.hpp"

namespace akv {

#define AKV_CHECK_LAUNCH(name)                                                              \
  do {                                                                                      \
    hipError_t e_ = hipGetLastError();                                                      \
    if (e_ != hipSuccess) return fail(ANCHORKV_E_HIP, "%s: %s", name, hipGetErrorString(e_)); \
  } while (0)

constexpr int kMaxG = 16;

// S[g][a] = <q_g, k_a> * log2(e)/sqrt(D); qsum[g][grp] = sum of q over the group, same scale.
template <int DT>
__global__ __launch_bounds__(256) void k_dec_stab(const void* qv, const uint8_t* cache, int64_t stride, int64_t off_ak,
                                                 float* stab, float* qsum, int H, int G, int A, float c) {
  using T = typename Elem<DT>::T;
  constexpr int D = kHeadDim;
  __shared__ float qs[kMaxG * D];
  const int h = blockIdx.x % H, u = blockIdx.x / H;
  const int64_t uh = (int64_t)u * H + h;
  const T* q = reinterpret_cast<const T*>(qv) + uh * G * D;
  for (int i = threadIdx.x; i < G * D; i += blockDim.x) qs[i] = Elem<DT>::f(q[i]);
  __syncthreads();
  const T* AK = reinterpret_cast<const T*>(cache + (int64_t)u * stride + off_ak) + (int64_t)h * A * D;
  for (int i = threadIdx.x; i < G * A; i += blockDim.x) {
    const int g = i / A, a = i % A;
    const T* kr = AK + (int64_t)a * D;
    float s = 0.0f;
    for (int d = 0; d < D; ++d) s = fmaf(qs[g * D + d], Elem<DT>::f(kr[d]), s);
    stab[uh * G * A + i] = s * c;
  }
  for (int i = threadIdx.x; i < G * 4; i += blockDim.x) {
    const int g = i / 4, grp = i % 4;
    float s = 0.0f;
    for (int d = 0; d < 32; ++d) s += qs[g * D + grp * 32 + d];
    qsum[uh * G * 4 + i] = s * c;
  }
}

__device__ __forceinline__ void decode_record(const uint8_t* rec, float* r /*[128]*/) {
  uint16_t w[16];
  uint32_t sz[4];
  const uint4* p = reinterpret_cast<const uint4*>(rec);
  uint4 a = p[0], b = p[1], c = p[2];
  __builtin_memcpy(w, &a, 16);
  __builtin_memcpy(w + 8, &b, 16);
  __builtin_memcpy(sz, &c, 16);
  for (int j = 0; j < 16; ++j)
    for (int cc = 0; cc < 8; ++cc) {
      const int d = j + 16 * cc;
      const int g = d >> 5;
      const float sc = h2f((uint16_t)(sz[g] & 0xFFFFu)), z = h2f((uint16_t)(sz[g] >> 16));
      r[d] = fmaf(sc, (float)((w[j] >> (2 * cc)) & 3u), z);
    }
}

template <int DT>
__global__ __launch_bounds__(256) void k_dec_stream(const void* qv, const uint8_t* cache, int64_t stride,
                                                   int64_t off_words, int64_t off_rk, int64_t off_rv, int64_t off_ck,
                                                   int64_t off_cv, const float* stab, float2* part_ml, float* part_w,
                                                   float* part_acc, int H, int G, int N, int A, int C, int S2,
                                                   float c) {
  using T = typename Elem<DT>::T;
  constexpr int D = kHeadDim;
  extern __shared__ float dsm[];
  float* S = dsm;                 // [G][A]
  float* w = S + G * A;           // [G][A]
  float* acc = w + G * A;         // [G][D]
  float* qsc = acc + G * D;       // [G][D]
  __shared__ float m_run[kMaxG], scale[kMaxG], tmax_w[4][kMaxG];
  __shared__ int cnt_w[2][4];
  __shared__ int any_rescale;

  int bid = blockIdx.x;
  const int s = bid % S2; bid /= S2;
  const int h = bid % H;
  const int u = bid / H;
  const int64_t uh = (int64_t)u * H + h;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cps = (C + S2 - 1) / S2;
  const int c0 = s * cps, c1 = min(C, c0 + cps);
  const int t_beg = c0 * kChunk, t_end = min(N, c1 * kChunk);
  const uint8_t* base = cache + (int64_t)u * stride;
  const T* q = reinterpret_cast<const T*>(qv) + uh * G * D;

  for (int i = threadIdx.x; i < G * A; i += blockDim.x) { S[i] = stab[uh * G * A + i]; w[i] = 0.0f; }
  for (int i = threadIdx.x; i < G * D; i += blockDim.x) { acc[i] = 0.0f; qsc[i] = Elem<DT>::f(q[i]) * c; }
  if (threadIdx.x < kMaxG) m_run[threadIdx.x] = -INFINITY;
  __syncthreads();

  const uint32_t* words = reinterpret_cast<const uint32_t*>(base + off_words) + (int64_t)h * N * 2;
  int recK = 0, recV = 0;
  if (c0 < C) {
    recK = reinterpret_cast<const int*>(base + off_ck)[h * C + c0];
    recV = reinterpret_cast<const int*>(base + off_cv)[h * C + c0];
  }
  float lp[kMaxG];
  for (int g = 0; g < kMaxG; ++g) lp[g] = 0.0f;

  for (int tb = t_beg; tb < t_end; tb += blockDim.x) {
    const int t = tb + threadIdx.x;
    const bool valid = t < t_end;
    uint2 wd = valid ? reinterpret_cast<const uint2*>(words)[t] : make_uint2(0, 0);
    const int aK = wd.x & 0x7FFF, aV = wd.y & 0x7FFF;
    const bool fK = valid && (wd.x & 0x8000u), fV = valid && (wd.y & 0x8000u);
    const float gK = h2f((uint16_t)(wd.x >> 16)), gV = h2f((uint16_t)(wd.y >> 16));
    // ranks of flagged tokens within the tile (block-wide, in token order)
    const unsigned long long bK = __ballot(fK), bV = __ballot(fV);
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    if (lane == 0) { cnt_w[0][wave] = __popcll(bK); cnt_w[1][wave] = __popcll(bV); }
    __syncthreads();
    int preK = 0, preV = 0, totK = 0, totV = 0;
    for (int wv = 0; wv < 4; ++wv) {
      if (wv < wave) { preK += cnt_w[0][wv]; preV += cnt_w[1][wv]; }
      totK += cnt_w[0][wv]; totV += cnt_w[1][wv];
    }
    const int rk = recK + preK + __popcll(bK & below);
    const int rv = recV + preV + __popcll(bV & below);

    float sl[kMaxG];
    for (int g = 0; g < G; ++g) sl[g] = valid ? gK * S[g * A + aK] : -INFINITY;
    if (fK) {
      float r[D];
      decode_record(base + off_rk + (int64_t)rk * kRecBytes, r);
      for (int g = 0; g < G; ++g) {
        float dsum = 0.0f;
        for (int d = 0; d < D; ++d) dsum = fmaf(qsc[g * D + d], r[d], dsum);
        sl[g] += dsum;
      }
    }
    // tile max per q-head, lazy rescale when it grows by more than 2^8
    for (int g = 0; g < G; ++g) {
      const float mx = wave_max(sl[g]);
      if (lane == 0) tmax_w[wave][g] = mx;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      int any = 0;
      for (int g = 0; g < G; ++g) {
        const float tm = fmaxf(fmaxf(tmax_w[0][g], tmax_w[1][g]), fmaxf(tmax_w[2][g], tmax_w[3][g]));
        float f = 1.0f;
        if (tm > m_run[g] + 8.0f) {
          f = (m_run[g] == -INFINITY) ? 0.0f : exp2_fast(m_run[g] - tm);
          m_run[g] = tm;
          any = 1;
        }
        scale[g] = f;
      }
      any_rescale = any;
    }
    __syncthreads();
    if (any_rescale) {
      for (int i = threadIdx.x; i < G * A; i += blockDim.x) w[i] *= scale[i / A];
      for (int i = threadIdx.x; i < G * D; i += blockDim.x) acc[i] *= scale[i / D];
      for (int g = 0; g < G; ++g) lp[g] *= scale[g];
      __syncthreads();
    }
    float p[kMaxG];
    for (int g = 0; g < G; ++g) {
      p[g] = valid ? exp2_fast(sl[g] - m_run[g]) : 0.0f;
      lp[g] += p[g];
      if (valid) atomicAdd(&w[g * A + aV], p[g] * gV);
    }
    if (fV) {
      float r[D];
      decode_record(base + off_rv + (int64_t)rv * kRecBytes, r);
      for (int d = 0; d < D; ++d)
        for (int g = 0; g < G; ++g) atomicAdd(&acc[g * D + d], p[g] * r[d]);
    }
    recK += totK;
    recV += totV;
    __syncthreads();
  }
  // write this range's state
  for (int g = 0; g < G; ++g) {
    const float l = wave_sum(lp[g]);
    if (lane == 0) tmax_w[wave][g] = l;
  }
  __syncthreads();
  const int64_t ps = uh * S2 + s;
  if (threadIdx.x < G) {
    const int g = threadIdx.x;
    part_ml[ps * G + g] = make_float2(m_run[g], tmax_w[0][g] + tmax_w[1][g] + tmax_w[2][g] + tmax_w[3][g]);
  }
  for (int i = threadIdx.x; i < G * A; i += blockDim.x) part_w[ps * G * A + i] = w[i];
  for (int i = threadIdx.x; i < G * D; i += blockDim.x) part_acc[ps * G * D + i] = acc[i];
}

template <int DT>
__global__ __launch_bounds__(256) void k_dec_combine(const uint8_t* cache, int64_t stride, int64_t off_av,
                                                    const float2* part_ml, const float* part_w,
                                                    const float* part_acc, float* o, int H, int G, int A, int S2) {
  using T = typename Elem<DT>::T;
  constexpr int D = kHeadDim;
  extern __shared__ float f_s[];  // [G][S2]
  __shared__ float Linv[kMaxG];
  const int h = blockIdx.x % H, u = blockIdx.x / H;
  const int64_t uh = (int64_t)u * H + h;
  if (threadIdx.x < G) {
    const int g = threadIdx.x;
    float M = -INFINITY;
    for (int s = 0; s < S2; ++s) M = fmaxf(M, part_ml[(uh * S2 + s) * G + g].x);
    float L = 0.0f;
    for (int s = 0; s < S2; ++s) {
      const float2 v = part_ml[(uh * S2 + s) * G + g];
      const float f = v.x == -INFINITY ? 0.0f : exp2_fast(v.x - M);
      f_s[g * S2 + s] = f;
      L += f * v.y;
    }
    Linv[g] = 1.0f / L;
  }
  __syncthreads();
  const T* AV = reinterpret_cast<const T*>(cache + (int64_t)u * stride + off_av) + (int64_t)h * A * D;
  for (int i = threadIdx.x; i < G * D; i += blockDim.x) {
    const int g = i / D, d = i % D;
    float acc = 0.0f;
    for (int s = 0; s < S2; ++s) acc = fmaf(f_s[g * S2 + s], part_acc[((uh * S2 + s) * G + g) * D + d], acc);
    for (int a = 0; a < A; ++a) {
      float wa = 0.0f;
      for (int s = 0; s < S2; ++s) wa = fmaf(f_s[g * S2 + s], part_w[((uh * S2 + s) * G + g) * A + a], wa);
      acc = fmaf(wa, Elem<DT>::f(AV[(int64_t)a * D + d]), acc);
    }
    o[(uh * G + g) * D + d] = acc * Linv[g];
  }
}

template <int DT>
static int decode_impl(const anchorkv_plan_info& p, const void* cache_v, const void* q, float* o, void* ws_v,
                       hipStream_t st) {
  const uint8_t* cache = reinterpret_cast<const uint8_t*>(cache_v);
  uint8_t* ws = reinterpret_cast<uint8_t*>(ws_v);
  const DecodeWs w = decode_ws_layout(p);
  const int U = p.units, H = p.H, G = p.G, A = p.A, N = p.N, C = p.n_chunks, S2 = w.S2;
  if (G > kMaxG) return fail(ANCHORKV_E_SHAPE, "decode supports q_per_kv <= %d", kMaxG);
  const size_t lds = sizeof(float) * (2 * (size_t)G * A + 2 * (size_t)G * kHeadDim);
  if (lds > 150 * 1024) return fail(ANCHORKV_E_SHAPE, "decode: q_per_kv * anchors too large for LDS");
  const float c = kLog2e / sqrtf((float)kHeadDim);
  float* stab = reinterpret_cast<float*>(ws + w.stab);
  float* qsum = reinterpret_cast<float*>(ws + w.qsum);
  prof_call_begin(st);
  k_dec_stab<DT><<<(unsigned)(U * H), 256, 0, st>>>(q, cache, p.unit_stride, p.off_anchor_k, stab, qsum, H, G, A, c);
  AKV_CHECK_LAUNCH("k_dec_stab");
  prof_mark(st, "dec_stab");
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(&k_dec_stream<DT>), hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)lds) != hipSuccess)
    return fail(ANCHORKV_E_HIP, "decode: cannot raise the dynamic LDS limit");
  k_dec_stream<DT><<<(unsigned)((int64_t)U * H * S2), 256, lds, st>>>(
      q, cache, p.unit_stride, p.off_words, p.off_res_k, p.off_res_v, p.off_chunk_k, p.off_chunk_v, stab,
      reinterpret_cast<float2*>(ws + w.part_ml), reinterpret_cast<float*>(ws + w.part_w),
      reinterpret_cast<float*>(ws + w.part_acc), H, G, N, A, C, S2, c);
  AKV_CHECK_LAUNCH("k_dec_stream");
  prof_mark(st, "dec_stream");
  k_dec_combine<DT><<<(unsigned)(U * H), 256, sizeof(float) * G * S2, st>>>(
      cache, p.unit_stride, p.off_anchor_v, reinterpret_cast<const float2*>(ws + w.part_ml),
      reinterpret_cast<const float*>(ws + w.part_w), reinterpret_cast<const float*>(ws + w.part_acc), o, H, G, A, S2);
  AKV_CHECK_LAUNCH("k_dec_combine");
  prof_mark(st, "dec_combine");
  return 0;
}

int run_decode(const anchorkv_plan_info& p, const void* cache, const void* q, float* o, void* ws, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (p.dtype == ANCHORKV_BF16) return decode_impl<ANCHORKV_BF16>(p, cache, q, o, ws, st);
  return decode_impl<ANCHORKV_F32>(p, cache, q, o, ws, st);
}

}  // namespace akv
