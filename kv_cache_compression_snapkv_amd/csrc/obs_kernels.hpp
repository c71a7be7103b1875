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
};

template <int DT> struct ObsCfg {
  using T = typename Elem<DT>::T;
  static constexpr int D = kHeadDim;
  static constexpr int PAD = DT == ANCHORKV_BF16 ? 8 : 4;  // row padding (elements) against bank conflicts
  static constexpr int LDK = D + PAD;                      // row stride of [key][D] tiles
  static constexpr int LDVT = 64 + (DT == ANCHORKV_BF16 ? 8 : 4);  // row stride of the transposed V tile
  static constexpr int NSTEP = D / Mfma<DT>::KSTEP;
};

template <int DT, int MODE, int QPW>
__global__ __launch_bounds__(512) void k_obs(ObsArgs a) {
  using C = ObsCfg<DT>;
  using T = typename C::T;
  using M = Mfma<DT>;
  using frag = typename M::frag;
  constexpr int D = C::D, LDK = C::LDK, NSTEP = C::NSTEP, LDVT = C::LDVT;

  __shared__ __attribute__((aligned(16))) T Ks[64 * LDK];
  __shared__ __attribute__((aligned(16))) T Vs[(MODE == OBS_STATS) ? 16 : (MODE == OBS_SCORE ? D * LDVT : 64 * LDK)];
  __shared__ __attribute__((aligned(16))) T Gs[(MODE == OBS_UTIL) ? 64 * LDK : 16];
  __shared__ float colpart[8][64];
  __shared__ float vv_s[64];
  __shared__ float gam_s[64];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int col = lane & 15, kg = lane >> 4;
  int bid = blockIdx.x;
  const int s = bid % a.S1; bid /= a.S1;
  const int h = bid % a.H;
  const int u = bid / a.H;
  const int N = a.N, H = a.H;
  const int k0 = s * a.kps;
  const int k1 = min(N, k0 + a.kps);
  const int64_t uh = (int64_t)u * H + h;
  const T* Kp = reinterpret_cast<const T*>(a.K) + uh * N * D;
  const T* Vp = reinterpret_cast<const T*>(a.V) + uh * N * D;
  const T* Qp = reinterpret_cast<const T*>(a.Q) + ((int64_t)u * H * a.G + (int64_t)h * a.G) * a.n_obs * D;

  // ---- per-wave query blocks and their B fragments (constant over all keys)
  frag qf[QPW][NSTEP];
  frag ofh[(MODE == OBS_UTIL) ? QPW : 1][NSTEP];
  frag ofl[(MODE == OBS_UTIL && DT == ANCHORKV_BF16) ? QPW : 1][NSTEP];
  float mq[QPW], il[QPW], ooq[QPW];
  bool qvalid[QPW];
  int qj[QPW];
  for (int qi = 0; qi < QPW; ++qi) {
    const int qb = wave + qi * nw;
    const int q = qb * 16 + col;
    qvalid[qi] = (qb * 16 < a.GQp) && q < a.GQ;
    qj[qi] = q % a.n_obs;
    for (int st = 0; st < NSTEP; ++st) {
      const int kk = st * M::KSTEP + kg * M::KW;
      qf[qi][st] = qvalid[qi] ? M::load(Qp + (int64_t)q * D + kk) : M::zero();
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

  for (int t0 = k0; t0 < k1; t0 += 64) {
    // ---- stage the key tile (and value / gathered-anchor tiles)
    constexpr int EPC = 16 / sizeof(T);  // elements per 16-byte chunk
    constexpr int CPR = D / EPC;          // chunks per row
    for (int ch = threadIdx.x; ch < 64 * CPR; ch += blockDim.x) {
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
    if constexpr (MODE == OBS_SCORE) {
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
    if constexpr (MODE == OBS_UTIL) {
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
      frag af[2][NSTEP];
      frag gf[(MODE == OBS_UTIL) ? 2 : 1][NSTEP];
      frag vf[(MODE == OBS_UTIL) ? 2 : 1][NSTEP];
      for (int k2 = 0; k2 < 2; ++k2) {
        const int row = (c2 * 2 + k2) * 16 + col;
        for (int st = 0; st < NSTEP; ++st) {
          const int kk = st * M::KSTEP + kg * M::KW;
          af[k2][st] = M::load(&Ks[row * LDK + kk]);
          if constexpr (MODE == OBS_UTIL) {
            gf[k2][st] = M::load(&Gs[row * LDK + kk]);
            vf[k2][st] = M::load(&Vs[row * LDK + kk]);
          }
        }
      }
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
        if (!(wave + qi * nw < a.GQp / 16)) continue;  // wave-uniform
        float pv[2][4];
        for (int k2 = 0; k2 < 2; ++k2) {
          const int kb = c2 * 2 + k2;
          f32x4 acc = {0, 0, 0, 0}, accg = {0, 0, 0, 0}, accv = {0, 0, 0, 0};
          for (int st = 0; st < NSTEP; ++st) acc = M::mma(af[k2][st], qf[qi][st], acc);
          if constexpr (MODE == OBS_UTIL) {
            for (int st = 0; st < NSTEP; ++st) accg = M::mma(gf[k2][st], qf[qi][st], accg);
            for (int st = 0; st < NSTEP; ++st) accv = M::mma(vf[k2][st], ofh[qi][st], accv);
            if constexpr (DT == ANCHORKV_BF16)
              for (int st = 0; st < NSTEP; ++st) accv = M::mma(vf[k2][st], ofl[qi][st], accv);
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
                    const int q = (wave + qi * nw) * 16 + col;
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
      // column sums over the 16 query lanes, then over waves in a fixed order
      for (int kb = 0; kb < 4; ++kb)
        for (int r = 0; r < 4; ++r) {
          float v = colsum[kb][r];
          v += __shfl_xor(v, 1, 64);
          v += __shfl_xor(v, 2, 64);
          v += __shfl_xor(v, 4, 64);
          v += __shfl_xor(v, 8, 64);
          if (col == 0) colpart[wave][kb * 16 + kg * 4 + r] = v;
        }
      __syncthreads();
      if (threadIdx.x < 64) {
        const int t = t0 + threadIdx.x;
        float v = 0.0f;
        for (int w = 0; w < nw; ++w) v += colpart[w][threadIdx.x];
        if (t < k1) {
          if constexpr (MODE == OBS_SCORE) {
            a.score[uh * N + t] = v;
          } else {
            const bool anc = a.anchor_of[uh * N + t] >= 0;
            const int64_t iK = ((int64_t)u * 2 * H + h) * N + t;
            a.util[iK] = anc ? -1.0f : v;
          }
        }
      }
    }
    __syncthreads();
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
      const int qb = wave + qi * nw;
      if (kg == 0 && qb * 16 < a.GQp) a.ml_part[(uh * a.S1 + s) * a.GQp + qb * 16 + col] = make_float2(m, l);
    }
  }
  if constexpr (MODE == OBS_SCORE) {
    for (int qi = 0; qi < QPW; ++qi) {
      const int qb = wave + qi * nw;
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
