// Observation-window kernels of the compression pass (gfx950, MFMA).
//
// One workgroup per (unit, KV head, key split); its waves split the padded
// observation queries into 16-column blocks.  Every kernel computes the
// transposed logit tile S^T[key][query] = K Q^T on MFMA (exact bf16 or f32
// operands, f32 accumulation), 64 keys per step, and differs in what it does
// with it:
//   STATS: running max / sum-exp per query (softmax statistics).
//   SCORE: p = exp(s - m)/l; column sums over queries (anchor score, Pith
//          review "What carries the argument": SnapKV observation-window
//          score pooled over GQA heads) and o = P V (PV on MFMA, p split into
//          bf16 hi + lo so the product keeps ~16 bits).
//   UTIL:  first-order output-error utility of every key (Pith review,
//          "Assumptions & free parameters": key channel
//          p |<q, r_K>|/sqrt(D) ||v - o||), with <q, r_K> = <q, k_t> -
//          gamma_t <q, k_a(t)> (both exact-operand MFMA) and ||v - o||^2 =
//          ||v||^2 - 2<v, o> + ||o||^2 (o split hi + lo), recomputed directly
//          when cancellation could cost precision.  (The value channel
//          score_t ||r_V|| is written by the assignment kernel.)
// Query j of a q-head sits at position N - n_obs + j and sees keys t <=
// N - n_obs + j.
#pragma once

#include "device_common.hpp"

namespace akv {

enum { OBS_STATS = 0, OBS_SCORE = 1, OBS_UTIL = 2, OBS_UTILX = 3 };

struct ObsArgs {
  const void* K;
  const void* V;
  const void* Q;
  const uint8_t* cache;
  int64_t stride, off_anchor_k;
  float2* ml_part;
  const float2* ml;
  float* o_part;
  const uint16_t* ohl;   // bf16 hi/lo of o [U][H][2][GQp][D]
  const float* ofull;    // f32 o [U][H][GQp][D]
  const float* oo;       // ||o||^2 [U][H][GQp]
  float* score;
  const float* gam;      // [U][2][H][N]
  const int* aidx;       // [U][2][H][N]
  const float* rn2;      // [U][2][H][N]
  const int* anchor_of;  // [U][H][N]
  const float* vn2;      // [U][H][N] ||v_t||^2
  float* util;           // [U][2][H][N]
  uint8_t* uflag;        // [U][H][nflag] UTIL tile flags (bf16 path): 1 = recompute in UTILX
  int nflag;             // tile flags per (unit, head)
  int U, H, G, N, n_obs, GQ, GQp, S1, kps, A;
  int S1u, kps_u;         // key splits of the pipelined UTIL kernel (<= 2048 keys each)
  float c;               // log2(e)/sqrt(D)
  float inv_sqrt_d;
  const float2* rope_cs; // pre-RoPE keys: (cos, sin) [N][D/2] of the rotation at each position
  int qsplit;            // generic kernel: query-block groups per (unit, head, key split), each its own
                         // block of 8 query blocks; > 1 adds the groups' score / key-utility partials
};

template <int DT> struct ObsCfg {
  using T = typename Elem<DT>::T;
  static constexpr int D = kHeadDim;
  static constexpr int PAD = DT == ANCHORKV_BF16 ? 8 : 4;  // row padding (elements) against bank conflicts
  static constexpr int LDK = D + PAD;                      // row stride of [key][D] tiles
  static constexpr int LDVT = 64 + (DT == ANCHORKV_BF16 ? 8 : 4);  // row stride of the transposed V tile
  static constexpr int NSTEP = D / Mfma<DT>::KSTEP;
};

// Four consecutive elements of a row as floats (bf16: 8-byte load, f32:
// 16-byte load; the caller keeps the address aligned to that size).
template <int SRC> __device__ __forceinline__ void ld4f(const typename Elem<SRC>::T* p, float (&o)[4]) {
  if constexpr (SRC == ANCHORKV_BF16) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    o[0] = __uint_as_float(v.x << 16); o[1] = __uint_as_float(v.x & 0xFFFF0000u);
    o[2] = __uint_as_float(v.y << 16); o[3] = __uint_as_float(v.y & 0xFFFF0000u);
  } else {
    const float4 v = *reinterpret_cast<const float4*>(p);
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
  }
}

// Rotary embedding of coordinates i0..i0+3 (x0) and their partners
// 64+i0..64+i0+3 (x1) with (cos, sin) of the position: (x0, x1) ->
// (x0 cos - x1 sin, x0 sin + x1 cos).
__device__ __forceinline__ void rope4(float (&x0)[4], float (&x1)[4], const float2* cs) {
  const float4 ca = reinterpret_cast<const float4*>(cs)[0], cb = reinterpret_cast<const float4*>(cs)[1];
  const float c[4] = {ca.x, ca.z, cb.x, cb.z}, s[4] = {ca.y, ca.w, cb.y, cb.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = x0[i], b = x1[i];
    x0[i] = fmaf(a, c[i], -b * s[i]);
    x1[i] = fmaf(a, s[i], b * c[i]);
  }
}

// DT: the arithmetic (tile and MFMA) type; SRC: the storage type of K, V, Q
// and the cache's anchors (== DT except with pre-RoPE keys in f32
// arithmetic); ROPE: K holds pre-RoPE keys (Pith review, "Assumptions & free
// parameters": R_t is a per-position orthogonal map), rotated here at their
// positions while the tile is staged, and in UTIL the gathered anchor row of
// each token is rotated at the token's position, so <q, R_t k_t> -
// gamma_t <q, R_t k_a(t)> = <q, R_t r_t>.  In bf16 arithmetic the rotated
// rows are kept as bf16 hi + lo (two tiles, two MFMAs per step; about 16
// significant bits), the queries and values stay exact.
template <int DT, int MODE, int QPW, int SRC = DT, bool ROPE = false>
__global__ __launch_bounds__(512) void k_obs(ObsArgs a) {
  using C = ObsCfg<DT>;
  using T = typename C::T;
  using S = typename Elem<SRC>::T;
  using M = Mfma<DT>;
  using frag = typename M::frag;
  constexpr int D = C::D, LDK = C::LDK, NSTEP = C::NSTEP, LDVT = C::LDVT;
  static_assert(SRC == DT || (ROPE && DT == ANCHORKV_F32), "storage differs from arithmetic only for pre-RoPE keys");
  constexpr bool SPLIT = ROPE && DT == ANCHORKV_BF16;   // rotated rows as bf16 hi + lo

  __shared__ __attribute__((aligned(16))) T Ks[64 * LDK];
  __shared__ __attribute__((aligned(16))) T Vs[(MODE == OBS_STATS) ? 16 : (MODE == OBS_SCORE ? D * LDVT : 64 * LDK)];
  __shared__ __attribute__((aligned(16))) T Gs[(MODE == OBS_UTIL) ? 64 * LDK : 16];
  __shared__ __attribute__((aligned(16))) T Ks2[SPLIT ? 64 * LDK : 8];                        // lo parts
  __shared__ __attribute__((aligned(16))) T Gs2[(SPLIT && MODE == OBS_UTIL) ? 64 * LDK : 8];
  __shared__ float colpart[2][8][64];   // per tile parity: the waves' column sums
  __shared__ float vv_s[64];
  __shared__ float gam_s[64];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int col = lane & 15, kg = lane >> 4;
  int bid = blockIdx.x;
  const int s = bid % a.S1; bid /= a.S1;
  // query-block group of this block: blocks 0..nw-1 of the padded queries,
  // then nw..2nw-1, ... (more than 8 query blocks take several workgroups)
  int qgrp = 0;
  if (a.qsplit > 1) { qgrp = bid % a.qsplit; bid /= a.qsplit; }
  const int qbase = qgrp * nw;
  const bool qadd = a.qsplit > 1;   // partials of several groups are added
  const int h = bid % a.H;
  const int u = bid / a.H;
  const int N = a.N, H = a.H;
  const int k0 = s * a.kps;
  const int k1 = min(N, k0 + a.kps);
  const int64_t uh = (int64_t)u * H + h;
  const S* Kp = reinterpret_cast<const S*>(a.K) + uh * N * D;
  const S* Vp = reinterpret_cast<const S*>(a.V) + uh * N * D;
  const S* Qp = reinterpret_cast<const S*>(a.Q) + ((int64_t)u * H * a.G + (int64_t)h * a.G) * a.n_obs * D;

  // ---- per-wave query blocks and their B fragments (constant over all keys)
  frag qf[QPW][NSTEP];
  frag ofh[(MODE == OBS_UTIL) ? QPW : 1][NSTEP];
  frag ofl[(MODE == OBS_UTIL && DT == ANCHORKV_BF16) ? QPW : 1][NSTEP];
  float mq[QPW], il[QPW], ooq[QPW];
  bool qvalid[QPW];
  int qj[QPW];
  for (int qi = 0; qi < QPW; ++qi) {
    const int qb = qbase + wave + qi * nw;
    const int q = qb * 16 + col;
    qvalid[qi] = (qb * 16 < a.GQp) && q < a.GQ;
    qj[qi] = q % a.n_obs;
    for (int st = 0; st < NSTEP; ++st) {
      const int kk = st * M::KSTEP + kg * M::KW;
      if constexpr (SRC == DT) qf[qi][st] = qvalid[qi] ? M::load(Qp + (int64_t)q * D + kk) : M::zero();
      else qf[qi][st] = qvalid[qi] ? Elem<SRC>::f(Qp[(int64_t)q * D + kk]) : M::zero();
      if constexpr (MODE == OBS_UTIL) {
        if constexpr (DT == ANCHORKV_BF16) {
          const uint16_t* oh = a.ohl + (uh * 2 + 0) * a.GQp * D;
          const uint16_t* ol = a.ohl + (uh * 2 + 1) * a.GQp * D;
          ofh[qi][st] = qvalid[qi] ? M::load(reinterpret_cast<const T*>(oh + (int64_t)q * D + kk)) : M::zero();
          ofl[qi][st] = qvalid[qi] ? M::load(reinterpret_cast<const T*>(ol + (int64_t)q * D + kk)) : M::zero();
        } else {
          ofh[qi][st] = qvalid[qi] ? a.ofull[(uh * a.GQp + q) * D + kk] : 0.0f;
        }
      }
    }
    mq[qi] = -INFINITY; il[qi] = 0.0f; ooq[qi] = 0.0f;
    if constexpr (MODE != OBS_STATS) {
      if (qvalid[qi]) {
        float2 v = a.ml[uh * a.GQp + q];
        mq[qi] = v.x; il[qi] = v.y;
      }
    }
    if constexpr (MODE == OBS_UTIL) {
      if (qvalid[qi]) ooq[qi] = a.oo[uh * a.GQp + q];
    }
  }
  (void)ooq;

  // running softmax stats (STATS) / PV accumulators (SCORE)
  float m_run[QPW], l_run[QPW];
  for (int qi = 0; qi < QPW; ++qi) { m_run[qi] = -INFINITY; l_run[qi] = 0.0f; }
  f32x4 oacc[(MODE == OBS_SCORE) ? QPW : 1][(MODE == OBS_SCORE) ? 8 : 1];
  if constexpr (MODE == OBS_SCORE)
    for (int qi = 0; qi < QPW; ++qi)
      for (int db = 0; db < 8; ++db) oacc[qi][db] = f32x4{0, 0, 0, 0};

  const int vis_base = N - a.n_obs;  // query j sees keys <= vis_base + j

  // ---- pre-RoPE staging, software-pipelined: item (row r, coordinates
  // i0..i0+3 and 64+i0..64+i0+3), RIT per thread (the block has 512 threads);
  // the rows of tile t0 + 64 (keys and their (cos, sin); in UTIL also values
  // and the tokens' anchor rows, whose indices come a tile earlier; in SCORE
  // the value tile) are loaded into registers while tile t0 is computed, and
  // rotated into the tile buffers after the tile's barrier
  using R4 = typename std::conditional<SRC == ANCHORKV_BF16, uint2, float4>::type;
  constexpr int RIT = ROPE ? 2 : 1;                                      // 64 x 16 items / 512 threads
  constexpr int VIT = (ROPE && MODE == OBS_SCORE) ? (SPLIT ? 2 : 4) : 1;  // transposed-value items
  struct RopeRaw { R4 k0, k1, g0, g1, v0, v1; float4 ca, cb; };
  RopeRaw rr[RIT];
  int ran[RIT];   // UTIL: anchor index of the item's token in the next tile load_raw reads
  uint4 vtr[VIT];   // SCORE: 16-byte value chunks (bf16) or 4 floats (f32) of the transposed tile
  auto r4f = [](const R4& x, float (&o)[4]) {
    if constexpr (SRC == ANCHORKV_BF16) {
      o[0] = __uint_as_float(x.x << 16); o[1] = __uint_as_float(x.x & 0xFFFF0000u);
      o[2] = __uint_as_float(x.y << 16); o[3] = __uint_as_float(x.y & 0xFFFF0000u);
    } else {
      o[0] = x.x; o[1] = x.y; o[2] = x.z; o[3] = x.w;
    }
  };
  auto load_raw = [&](int tb) {
#pragma unroll
    for (int k = 0; k < RIT; ++k) {
      const int it = threadIdx.x + k * 512;
      const int r = it >> 4, i0 = (it & 15) * 4;
      const int t = min(tb + r, k1 - 1);   // rows past the range repeat the last one (masked later)
      rr[k].k0 = *reinterpret_cast<const R4*>(Kp + (int64_t)t * D + i0);
      rr[k].k1 = *reinterpret_cast<const R4*>(Kp + (int64_t)t * D + 64 + i0);
      const float4* cs = reinterpret_cast<const float4*>(a.rope_cs + (int64_t)t * (D / 2) + i0);
      rr[k].ca = cs[0];
      rr[k].cb = cs[1];
      if constexpr (MODE == OBS_UTIL) {
        const S* ap = reinterpret_cast<const S*>(a.cache + (int64_t)u * a.stride + a.off_anchor_k) +
                      ((int64_t)h * a.A + ran[k]) * D;
        rr[k].g0 = *reinterpret_cast<const R4*>(ap + i0);
        rr[k].g1 = *reinterpret_cast<const R4*>(ap + 64 + i0);
        rr[k].v0 = *reinterpret_cast<const R4*>(Vp + (int64_t)t * D + i0);
        rr[k].v1 = *reinterpret_cast<const R4*>(Vp + (int64_t)t * D + 64 + i0);
        ran[k] = a.aidx[((int64_t)u * 2 * H + h) * N + min(tb + 64 + r, k1 - 1)];   // side 0 = K
      }
    }
    if constexpr (MODE == OBS_SCORE) {
#pragma unroll
      for (int k = 0; k < VIT; ++k) {
        // bf16: chunk (row ch % 64, 16-byte column ch / 64); f32: 4 floats
        const int ch = threadIdx.x + k * 512;
        const int r = ch % 64, c4 = ch / 64;
        const int t = min(tb + r, k1 - 1);
        vtr[k] = *reinterpret_cast<const uint4*>(Vp + (int64_t)t * D + c4 * (16 / (int)sizeof(S)));
      }
    }
  };
  // rotate the loaded rows of tile tb into the tile buffers (rows past the range: zeros)
  auto store_rot = [&](int tb) {
    // four rotated coordinates into a tile row: f32, or bf16 hi (and lo)
    auto put4 = [&](T* hi, T* lo, int off, const float (&x)[4]) {
      if constexpr (SPLIT) {
        uint16_t h4[4], l4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) { h4[i] = f2bf(x[i]); l4[i] = f2bf(x[i] - bf2f(h4[i])); }
        *reinterpret_cast<uint2*>(&hi[off]) = make_uint2(h4[0] | (uint32_t)h4[1] << 16, h4[2] | (uint32_t)h4[3] << 16);
        *reinterpret_cast<uint2*>(&lo[off]) = make_uint2(l4[0] | (uint32_t)l4[1] << 16, l4[2] | (uint32_t)l4[3] << 16);
      } else {
        (void)lo;
        *reinterpret_cast<float4*>(&hi[off]) = make_float4(x[0], x[1], x[2], x[3]);
      }
    };
#pragma unroll
    for (int k = 0; k < RIT; ++k) {
      const int it = threadIdx.x + k * 512;
      const int r = it >> 4, i0 = (it & 15) * 4;
      const bool ok = tb + r < k1;
      float2 cs[4] = {make_float2(rr[k].ca.x, rr[k].ca.y), make_float2(rr[k].ca.z, rr[k].ca.w),
                      make_float2(rr[k].cb.x, rr[k].cb.y), make_float2(rr[k].cb.z, rr[k].cb.w)};
      float x0[4], x1[4];
      r4f(rr[k].k0, x0);
      r4f(rr[k].k1, x1);
      rope4(x0, x1, cs);
      if (!ok)
#pragma unroll
        for (int i = 0; i < 4; ++i) { x0[i] = 0.0f; x1[i] = 0.0f; }
      put4(Ks, Ks2, r * LDK + i0, x0);
      put4(Ks, Ks2, r * LDK + 64 + i0, x1);
      if constexpr (MODE == OBS_UTIL) {
        float g0[4], g1[4];
        r4f(rr[k].g0, g0);
        r4f(rr[k].g1, g1);
        rope4(g0, g1, cs);
        if (!ok)
#pragma unroll
          for (int i = 0; i < 4; ++i) { g0[i] = 0.0f; g1[i] = 0.0f; }
        put4(Gs, Gs2, r * LDK + i0, g0);
        put4(Gs, Gs2, r * LDK + 64 + i0, g1);
        const R4 rv0 = rr[k].v0, rv1 = rr[k].v1;
        float v0[4], v1[4];
        r4f(rv0, v0);
        r4f(rv1, v1);
        if (!ok)
#pragma unroll
          for (int i = 0; i < 4; ++i) { v0[i] = 0.0f; v1[i] = 0.0f; }
        if constexpr (SPLIT) {
          // values stay exact bf16: 8-byte copies
          *reinterpret_cast<uint2*>(&Vs[r * LDK + i0]) = ok ? rv0 : make_uint2(0, 0);
          *reinterpret_cast<uint2*>(&Vs[r * LDK + 64 + i0]) = ok ? rv1 : make_uint2(0, 0);
        } else {
          *reinterpret_cast<float4*>(&Vs[r * LDK + i0]) = make_float4(v0[0], v0[1], v0[2], v0[3]);
          *reinterpret_cast<float4*>(&Vs[r * LDK + 64 + i0]) = make_float4(v1[0], v1[1], v1[2], v1[3]);
        }
        // ||v||^2 of the row: the 16 items of a row are 16 consecutive lanes
        float vv = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) vv = fmaf(v0[i], v0[i], fmaf(v1[i], v1[i], vv));
        vv = row_sum(vv);
        if ((it & 15) == 0) vv_s[r] = vv;
      }
    }
    if constexpr (MODE == OBS_SCORE) {
      // transposed value tile Vt[d][key]
#pragma unroll
      for (int k = 0; k < VIT; ++k) {
        const int ch = threadIdx.x + k * 512;
        const int r = ch % 64, c4 = ch / 64;
        const bool ok = tb + r < k1;
        constexpr int EPC4 = 16 / (int)sizeof(S);
        S tmp[EPC4];
        const uint4 raw = ok ? vtr[k] : make_uint4(0, 0, 0, 0);
        __builtin_memcpy(tmp, &raw, 16);
#pragma unroll
        for (int i = 0; i < EPC4; ++i) Vs[(c4 * EPC4 + i) * LDVT + r] = tmp[i];
      }
    }
  };
  // score / key utility of the keys of tile tb from the waves' column sums
  auto finish_tile = [&](int tb) {
    if (threadIdx.x < 64) {
      const int t = tb + threadIdx.x;
      float v = 0.0f;
      for (int w = 0; w < nw; ++w) v += colpart[((tb - k0) >> 6) & 1][w][threadIdx.x];
      if (t < k1) {
        // with query groups the two-or-more partials are added onto a zeroed
        // word (with two of them the sum does not depend on their order)
        if constexpr (MODE == OBS_SCORE) {
          if (qadd) atomicAdd(&a.score[uh * N + t], v);
          else a.score[uh * N + t] = v;
        } else {
          const bool anc = a.anchor_of[uh * N + t] >= 0;
          const int64_t iK = ((int64_t)u * 2 * H + h) * N + t;
          if (anc) a.util[iK] = -1.0f;
          else if (qadd) atomicAdd(&a.util[iK], v);
          else a.util[iK] = v;
        }
      }
    }
  };
  if constexpr (ROPE) {
    if constexpr (MODE == OBS_UTIL) {
#pragma unroll
      for (int k = 0; k < RIT; ++k) {
        const int r = (threadIdx.x + k * 512) >> 4;
        ran[k] = a.aidx[((int64_t)u * 2 * H + h) * N + min(k0 + r, k1 - 1)];
      }
    }
    load_raw(k0);
  }

  for (int t0 = k0; t0 < k1; t0 += 64) {
    // ---- stage the key tile (and value / gathered-anchor tiles)
    constexpr int EPC = 16 / sizeof(T);  // elements per 16-byte chunk
    constexpr int CPR = D / EPC;          // chunks per row
    if constexpr (ROPE) store_rot(t0);
    for (int ch = threadIdx.x; ch < (ROPE ? 0 : 64 * CPR); ch += blockDim.x) {
      const int r = ch / CPR, cc = ch % CPR;
      const int t = t0 + r;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (t < k1) v = *reinterpret_cast<const uint4*>(Kp + (int64_t)t * D + cc * EPC);
      *reinterpret_cast<uint4*>(&Ks[r * LDK + cc * EPC]) = v;
      if constexpr (MODE == OBS_UTIL) {
        uint4 w = make_uint4(0, 0, 0, 0);
        if (t < k1) w = *reinterpret_cast<const uint4*>(Vp + (int64_t)t * D + cc * EPC);
        *reinterpret_cast<uint4*>(&Vs[r * LDK + cc * EPC]) = w;
        uint4 g = make_uint4(0, 0, 0, 0);
        if (t < k1) {
          const int an = a.aidx[((int64_t)u * 2 * H + h) * N + t];  // side 0 = K
          const T* ap = reinterpret_cast<const T*>(a.cache + (int64_t)u * a.stride + a.off_anchor_k) + ((int64_t)h * a.A + an) * D;
          g = *reinterpret_cast<const uint4*>(ap + cc * EPC);
        }
        *reinterpret_cast<uint4*>(&Gs[r * LDK + cc * EPC]) = g;
      }
    }
    if constexpr (MODE == OBS_SCORE && !ROPE) {
      // transposed value tile Vt[d][key]; consecutive threads take consecutive keys
      for (int ch = threadIdx.x; ch < 64 * CPR; ch += blockDim.x) {
        const int r = ch % 64, cc = ch / 64;
        const int t = t0 + r;
        uint4 raw = make_uint4(0, 0, 0, 0);
        if (t < k1) raw = *reinterpret_cast<const uint4*>(Vp + (int64_t)t * D + cc * EPC);
        T tmp[EPC];
        __builtin_memcpy(tmp, &raw, 16);
        for (int i = 0; i < EPC; ++i) Vs[(cc * EPC + i) * LDVT + r] = tmp[i];
      }
    }
    if constexpr (MODE == OBS_UTIL) {
      if (threadIdx.x < 64) {
        const int t = t0 + threadIdx.x;
        gam_s[threadIdx.x] = t < k1 ? a.gam[((int64_t)u * 2 * H + h) * N + t] : 0.0f;
      }
    }
    __syncthreads();
    if constexpr (MODE != OBS_STATS) {
      if (t0 > k0) finish_tile(t0 - 64);
    }
    // pre-RoPE: the next tile's rows are loaded while this one is computed
    if constexpr (ROPE) {
      if (t0 + 64 < k1) load_raw(t0 + 64);
    }
    if constexpr (MODE == OBS_UTIL && !ROPE) {
      // ||v||^2 per key from the staged tile: 4 consecutive threads per key
      for (int kk = threadIdx.x >> 2; kk < 64; kk += blockDim.x >> 2) {
        const int part = threadIdx.x & 3;
        float vv = 0.0f;
        for (int d = part * (D / 4); d < (part + 1) * (D / 4); ++d) {
          const float x = Elem<DT>::f(Vs[kk * LDK + d]);
          vv = fmaf(x, x, vv);
        }
        vv += __shfl_xor(vv, 1, 64);
        vv += __shfl_xor(vv, 2, 64);
        if (part == 0) vv_s[kk] = vv;
      }
      __syncthreads();
    }

    float colsum[4][4];
    for (int kb = 0; kb < 4; ++kb)
      for (int r = 0; r < 4; ++r) colsum[kb][r] = 0.0f;

    for (int c2 = 0; c2 < 2; ++c2) {
      // value B-fragments of this 32-key chunk for the PV product
      frag vb[(MODE == OBS_SCORE) ? 8 : 1][(MODE == OBS_SCORE && DT == ANCHORKV_F32) ? 8 : 1];
      if constexpr (MODE == OBS_SCORE) {
        for (int db = 0; db < 8; ++db) {
          const int d = db * 16 + col;
          if constexpr (DT == ANCHORKV_BF16) {
            uint2 lo = *reinterpret_cast<const uint2*>(&Vs[d * LDVT + c2 * 32 + kg * 4]);
            uint2 hi = *reinterpret_cast<const uint2*>(&Vs[d * LDVT + c2 * 32 + 16 + kg * 4]);
            vb[db][0] = bits_to_frag(make_uint4(lo.x, lo.y, hi.x, hi.y));
          } else {
            for (int e = 0; e < 8; ++e)  // step e: key (2*c2 + e/4)*16 + 4*kg + e%4
              vb[db][e] = Vs[d * LDVT + (c2 * 2 + e / 4) * 16 + kg * 4 + (e % 4)];
          }
        }
      }
      for (int qi = 0; qi < QPW; ++qi) {
        if (!(qbase + wave + qi * nw < a.GQp / 16)) continue;  // wave-uniform
        float pv[2][4];
        for (int k2 = 0; k2 < 2; ++k2) {
          const int kb = c2 * 2 + k2;
          // A fragments of key block kb (one block at a time: fewer registers)
          frag af[NSTEP], gf[(MODE == OBS_UTIL) ? NSTEP : 1], vf[(MODE == OBS_UTIL) ? NSTEP : 1];
          frag af2[SPLIT ? NSTEP : 1], gf2[(SPLIT && MODE == OBS_UTIL) ? NSTEP : 1];
          {
            const int row = kb * 16 + col;
            for (int st = 0; st < NSTEP; ++st) {
              const int kk = st * M::KSTEP + kg * M::KW;
              af[st] = M::load(&Ks[row * LDK + kk]);
              if constexpr (SPLIT) af2[st] = M::load(&Ks2[row * LDK + kk]);
              if constexpr (MODE == OBS_UTIL) {
                gf[st] = M::load(&Gs[row * LDK + kk]);
                if constexpr (SPLIT) gf2[st] = M::load(&Gs2[row * LDK + kk]);
                vf[st] = M::load(&Vs[row * LDK + kk]);
              }
            }
          }
          f32x4 acc = {0, 0, 0, 0}, accg = {0, 0, 0, 0}, accv = {0, 0, 0, 0};
          for (int st = 0; st < NSTEP; ++st) acc = M::mma(af[st], qf[qi][st], acc);
          if constexpr (SPLIT)
            for (int st = 0; st < NSTEP; ++st) acc = M::mma(af2[st], qf[qi][st], acc);
          if constexpr (MODE == OBS_UTIL) {
            for (int st = 0; st < NSTEP; ++st) accg = M::mma(gf[st], qf[qi][st], accg);
            if constexpr (SPLIT)
              for (int st = 0; st < NSTEP; ++st) accg = M::mma(gf2[st], qf[qi][st], accg);
            for (int st = 0; st < NSTEP; ++st) accv = M::mma(vf[st], ofh[qi][st], accv);
            if constexpr (DT == ANCHORKV_BF16)
              for (int st = 0; st < NSTEP; ++st) accv = M::mma(vf[st], ofl[qi][st], accv);
          }
          for (int r = 0; r < 4; ++r) {
            const int kl = kb * 16 + kg * 4 + r;  // key within the tile
            const int t = t0 + kl;
            const bool valid = qvalid[qi] && t < k1 && t <= vis_base + qj[qi];
            const float sv = acc[r] * a.c;
            if constexpr (MODE == OBS_STATS) {
              pv[k2][r] = valid ? sv : -INFINITY;
            } else {
              float p = valid ? exp2_fast(sv - mq[qi]) * il[qi] : 0.0f;
              if constexpr (MODE == OBS_SCORE) {
                pv[k2][r] = p;
                colsum[kb][r] += p;
              } else {
                float term = 0.0f;
                if (p > 0.0f) {
                  const float qr = fabsf(acc[r] - gam_s[kl] * accg[r]) * a.inv_sqrt_d;
                  float vo2 = vv_s[kl] - 2.0f * accv[r] + ooq[qi];
                  if (vo2 < 0.5f * (vv_s[kl] + ooq[qi])) {  // cancellation: recompute directly
                    const int q = (qbase + wave + qi * nw) * 16 + col;
                    const float* orow = a.ofull + (uh * a.GQp + q) * D;
                    float acc2 = 0.0f;
                    for (int d = 0; d < D; ++d) {
                      const float df = Elem<DT>::f(Vs[kl * LDK + d]) - orow[d];
                      acc2 = fmaf(df, df, acc2);
                    }
                    vo2 = acc2;
                  }
                  term = p * qr * sqrtf(fmaxf(vo2, 0.0f));
                }
                colsum[kb][r] += term;
              }
            }
          }
        }
        if constexpr (MODE == OBS_STATS) {
          float mx = m_run[qi];
          for (int k2 = 0; k2 < 2; ++k2)
            for (int r = 0; r < 4; ++r) mx = fmaxf(mx, pv[k2][r]);
          if (mx > -INFINITY) {
            float l = l_run[qi] * exp2_fast(m_run[qi] - mx);
            for (int k2 = 0; k2 < 2; ++k2)
              for (int r = 0; r < 4; ++r) l += exp2_fast(pv[k2][r] - mx);
            m_run[qi] = mx;
            l_run[qi] = l;
          }
        }
        if constexpr (MODE == OBS_SCORE) {
          if constexpr (DT == ANCHORKV_BF16) {
            float p8[8];
            for (int e = 0; e < 8; ++e) p8[e] = pv[e / 4][e % 4];
            bf16x8 ph, pl;
            split8(p8, ph, pl);
            for (int db = 0; db < 8; ++db) {
              oacc[qi][db] = M::mma(ph, vb[db][0], oacc[qi][db]);
              oacc[qi][db] = M::mma(pl, vb[db][0], oacc[qi][db]);
            }
          } else {
            for (int db = 0; db < 8; ++db)
              for (int e = 0; e < 8; ++e) oacc[qi][db] = M::mma(pv[e / 4][e % 4], vb[db][e], oacc[qi][db]);
          }
        }
      }
    }

    if constexpr (MODE != OBS_STATS) {
      // column sums over the 16 query lanes; summed over the waves (fixed
      // order) after the next tile's staging barrier, or after the loop
      for (int kb = 0; kb < 4; ++kb)
        for (int r = 0; r < 4; ++r) {
          const float v = row_sum(colsum[kb][r]);   // over the 16 query lanes (DPP)
          if (col == 0) colpart[((t0 - k0) >> 6) & 1][wave][kb * 16 + kg * 4 + r] = v;
        }
    }
    __syncthreads();   // the tile's buffers are free; its column sums are published
  }
  if constexpr (MODE != OBS_STATS) {
    if (k1 > k0) finish_tile(k0 + ((k1 - k0 - 1) >> 6) * 64);
  }

  if constexpr (MODE == OBS_STATS) {
    for (int qi = 0; qi < QPW; ++qi) {
      float m = m_run[qi], l = l_run[qi];
      for (int o = 16; o <= 32; o <<= 1) {
        const float m2 = __shfl_xor(m, o, 64), l2 = __shfl_xor(l, o, 64);
        const float mx = fmaxf(m, m2);
        if (mx > -INFINITY) {
          l = l * exp2_fast(m - mx) + l2 * exp2_fast(m2 - mx);
          m = mx;
        }
      }
      const int qb = qbase + wave + qi * nw;
      if (kg == 0 && qb * 16 < a.GQp) a.ml_part[(uh * a.S1 + s) * a.GQp + qb * 16 + col] = make_float2(m, l);
    }
  }
  if constexpr (MODE == OBS_SCORE) {
    for (int qi = 0; qi < QPW; ++qi) {
      const int qb = qbase + wave + qi * nw;
      if (qb * 16 >= a.GQp) continue;
      for (int db = 0; db < 8; ++db)
        for (int r = 0; r < 4; ++r) {
          const int q = qb * 16 + kg * 4 + r;
          a.o_part[((uh * a.S1 + s) * a.GQp + q) * D + db * 16 + col] = oacc[qi][db][r];
        }
    }
  }
}

}  // namespace akv
