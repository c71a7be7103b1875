// Pipelined observation-window kernels for bf16 inputs (gfx950).
//
// Same modes as k_obs (STATS / SCORE / UTIL; see obs_kernels.hpp for what
// each computes and the page sections it follows), organised for latency
// hiding and a short per-element instruction stream:
//  * the block streams its key range in TK-key tiles (TK = 32 or 64) through
//    two LDS buffer sets; tiles are copied global -> LDS by asynchronous
//    global_load_lds_dwordx4 (16 bytes per lane, no registers) one tile
//    ahead of the one being computed; one barrier per tile;
//  * every [TK][128] bf16 tile is stored with its 16-byte chunks XOR-swizzled
//    per row, so that MFMA fragment reads (8 rows, same chunk) and the
//    transposing reads of the value tile (4 rows x 2 chunks) hit distinct
//    LDS banks;
//  * SCORE reads the P V operand with ds_read_b64_tr_b16, which hands each
//    lane 4 consecutive keys of one value coordinate straight from the
//    row-major tile;
//  * UTIL keeps the anchor index of every key of its range (<= 2048 keys) in
//    LDS, loaded once, so the gathered anchor rows can be copied ahead like
//    the key and value rows;
//  * 1/l is folded into the exponent offset (p = 2^(s c - m - log2 l)), so a
//    probability costs one FMA and one exp2; the causal / range mask is
//    applied only in tiles that reach past the first masked key;
//  * UTIL folds ||o||^2 into the accumulator of the <v, o> MFMA, so ||v - o||^2
//    costs one FMA.  Where that difference could cancel (below a quarter of
//    ||v||^2 + max ||o||^2) the tile is flagged; a second launch (UTILX)
//    recomputes only flagged tiles, evaluating ||v - o||^2 directly where the
//    expanded form loses precision;
//  * per-key sums over the block's query columns are reduced with DPP inside
//    a wave, written to a small LDS partial array, and combined across waves
//    one tile later (after the next barrier), in fixed wave order.
// The stage buffers are distinct __shared__ objects and the tile loop is
// unrolled by two, so the compiler can tell that compute-phase LDS reads do
// not alias the copies in flight and does not wait for them.
#pragma once

#include <type_traits>

#include "device_common.hpp"
#include "obs_kernels.hpp"

namespace akv {

#define AKV_LDS __attribute__((address_space(3)))

typedef short akv_v4s __attribute__((ext_vector_type(4)));

constexpr int kObsUtilMaxKeys = 2048;        // key range of one UTIL block
constexpr int kObsMaxWaves = 8;
constexpr int kObsSlot = 64;                 // per-key scalar / partial slots per tile (>= TK)

// Tile keys and stage buffers per mode.  Bytes in flight per compute unit
// (blocks x (ST-1) x tile bytes) set the achieved bandwidth: the loaded
// latency of an HBM copy is several microseconds.
template <int MODE, int QPW> struct ObsPipeCfg { static constexpr int TK = 64, ST = 2; };
template <int QPW> struct ObsPipeCfg<OBS_UTIL, QPW> { static constexpr int TK = 64, ST = 2; };
constexpr int kObsUtilTK = 64;   // UTIL / UTILX tile; the flag array allows >= 32
constexpr size_t kObsQaMaxBytes = 64 * 1024;   // largest <q, x_a> table of the UTIL fast pass
static_assert(ObsPipeCfg<OBS_UTIL, 1>::TK == kObsUtilTK && ObsPipeCfg<OBS_UTIL, 2>::TK == kObsUtilTK, "UTIL tile");

// Chunk swizzle of tile row r, a bijection of r & 15 onto 0..15 (LDS has 64
// banks of 4 bytes: 16 chunks of 16 bytes per cycle):
//  * a fragment read takes one logical chunk of 16 consecutive rows -> 16
//    distinct physical chunks;
//  * a transposing read takes logical chunks 2k, 2k+1 of 8 rows (r & 8
//    fixed) per 32-lane half -> f(r) >> 1 is distinct over those rows, so
//    the 16 (row, chunk) pairs land on 16 distinct chunks.
__device__ __forceinline__ int obs_swz(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }
// Physical chunk of logical chunk c (0..15) of tile row r.
__device__ __forceinline__ int obs_phys(int r, int c) { return r * 16 + (c ^ obs_swz(r)); }

// Asynchronous global -> LDS copies: lane l writes lds_base + size*l; the LDS
// base must be the same for the whole wave.
__device__ __forceinline__ void dma16(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds(src, (AKV_LDS void*)lds_base, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds(src, (AKV_LDS void*)lds_base, 4, 0, 0);
}

// s_waitcnt vmcnt(0) with the other counters untouched (gfx9 encoding:
// vmcnt bits 3:0 and 15:14, expcnt 6:4 = 7, lgkmcnt 11:8 = 15).  A builtin,
// unlike inline asm, is visible to the compiler's own wait-count tracking.
#define AKV_VMCNT_IMM(n) (((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(AKV_VMCNT_IMM(0)); }
// s_waitcnt vmcnt(n) for a wave-uniform n (the immediate must be a constant)
#define AKV_VM_CASE(n) case n: __builtin_amdgcn_s_waitcnt(AKV_VMCNT_IMM(n)); break;
__device__ __forceinline__ void wait_vm_le(int n) {
  switch (n) {
    AKV_VM_CASE(0) AKV_VM_CASE(1) AKV_VM_CASE(2) AKV_VM_CASE(3) AKV_VM_CASE(4) AKV_VM_CASE(5)
    AKV_VM_CASE(6) AKV_VM_CASE(7) AKV_VM_CASE(8) AKV_VM_CASE(9) AKV_VM_CASE(10) AKV_VM_CASE(11)
    AKV_VM_CASE(12) AKV_VM_CASE(13) AKV_VM_CASE(14) AKV_VM_CASE(15) AKV_VM_CASE(16) AKV_VM_CASE(17)
    AKV_VM_CASE(18) AKV_VM_CASE(19) AKV_VM_CASE(20) AKV_VM_CASE(21) AKV_VM_CASE(22) AKV_VM_CASE(23)
    AKV_VM_CASE(24) AKV_VM_CASE(25) AKV_VM_CASE(26) AKV_VM_CASE(27) AKV_VM_CASE(28) AKV_VM_CASE(29)
    AKV_VM_CASE(30) AKV_VM_CASE(31) AKV_VM_CASE(32) AKV_VM_CASE(33) AKV_VM_CASE(34) AKV_VM_CASE(35)
    AKV_VM_CASE(36) AKV_VM_CASE(37) AKV_VM_CASE(38) AKV_VM_CASE(39) AKV_VM_CASE(40) AKV_VM_CASE(41)
    AKV_VM_CASE(42) AKV_VM_CASE(43) AKV_VM_CASE(44) AKV_VM_CASE(45) AKV_VM_CASE(46) AKV_VM_CASE(47)
    AKV_VM_CASE(48) AKV_VM_CASE(49) AKV_VM_CASE(50) AKV_VM_CASE(51) AKV_VM_CASE(52) AKV_VM_CASE(53)
    AKV_VM_CASE(54) AKV_VM_CASE(55) AKV_VM_CASE(56) AKV_VM_CASE(57) AKV_VM_CASE(58) AKV_VM_CASE(59)
    AKV_VM_CASE(60) AKV_VM_CASE(61) AKV_VM_CASE(62)
    default: __builtin_amdgcn_s_waitcnt(AKV_VMCNT_IMM(0)); break;
  }
}
#undef AKV_VM_CASE

__device__ __forceinline__ bf16x8 lds_frag(const uint4* tile, int row, int c) {
  return bits_to_frag(tile[obs_phys(row, c)]);
}
// 4 consecutive keys (rows) of one value coordinate, via the transposing read.
__device__ __forceinline__ uint2 lds_tr(const uint4* tile, int row, int d) {
  const uint16_t* p = reinterpret_cast<const uint16_t*>(tile + obs_phys(row, d >> 3)) + (d & 7);
  akv_v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((AKV_LDS akv_v4s*)p);
  return __builtin_bit_cast(uint2, r);
}

// Tile copies: chunk-block jj (64 lanes, rows 4jj .. 4jj+3) of a [TK][128]
// tile.  Lane l writes physical chunk l & 15 of row r = 4jj + l/16, i.e.
// logical chunk (l & 15) ^ swz(r), with swz(4jj + rsub) = 8(jj & 1) + 2 rsub +
// ((jj >> 1) & 1).
struct DmaLane {
  int pc;     // lane & 15: physical chunk written
  int rsub;   // lane / 16: row within the 4-row block
  __device__ __forceinline__ explicit DmaLane(int lane) : pc(lane & 15), rsub(lane >> 4) {}
  // logical chunk this lane copies in chunk-block jj
  __device__ __forceinline__ int chunk(int jj) const { return pc ^ (8 * (jj & 1) + 2 * rsub + ((jj >> 1) & 1)); }
};

// Copy one [TK][128] tile of contiguous rows starting at `base` (rows beyond
// nval repeat row nval-1: valid memory, results masked).
template <int TK>
__device__ __forceinline__ int dma_rows(uint4* dst, const uint16_t* base, int nval, int nw, int wave,
                                         const DmaLane& dl) {
  int n = 0;
  for (int jj = wave; jj < TK / 4; jj += nw, ++n) {
    const int r = min(jj * 4 + dl.rsub, nval - 1);
    dma16(base + r * kHeadDim + dl.chunk(jj) * 8, dst + jj * 64);
  }
  return n;
}
// Copy one [TK][128] tile of gathered rows: row r is base + idx[r] * 128.
template <int TK>
__device__ __forceinline__ int dma_gather(uint4* dst, const uint16_t* base, const int* idx, int nval, int nw,
                                           int wave, const DmaLane& dl) {
  int n = 0;
  for (int jj = wave; jj < TK / 4; jj += nw, ++n) {
    const int r = min(jj * 4 + dl.rsub, nval - 1);
    dma16(base + (int64_t)idx[r] * kHeadDim + dl.chunk(jj) * 8, dst + jj * 64);
  }
  return n;
}

// One stage's LDS buffers.
struct ObsBufs {
  uint4* K;
  uint4* V;
  uint4* G;
  float* S;  // UTIL per-key scalars, kObsSlot each: [0] gamma_K, [1] ||v||^2, [2] anchor flag (int bits)
};

// ST: tile buffers (ST-1 tiles in flight while one is computed; UTILX uses 1).
// KS: key splits of a tile (UTIL): KS wave sets, each with every query block,
// take 1/KS of the tile's 16-key blocks, so that a block of 6 query blocks
// runs 12 waves (3 per SIMD) instead of 6 (2, 2, 1, 1); at most 6 query
// blocks with two splits.
// WPE: waves per SIMD the register allocation must allow.
// QAT (UTIL fast pass): <q, x_a> for every (observation query, anchor) of the
// head is computed once into an LDS table (dynamic shared memory, A rounded
// up to 16 rows of GQp floats) with the same MFMA sequence the per-key path
// uses, and gathered per key by its anchor index: no anchor-row copies, four
// fewer MFMAs and fragment reads per 16 keys.  For heads whose table fits.
template <int MODE, int QPW, int TK, int ST, int KS, int WPE, bool QAT = false>
__global__ __launch_bounds__(KS == 1 ? 512 : 768) __attribute__((amdgpu_waves_per_eu(WPE))) void k_obs_pipe(ObsArgs a) {
  constexpr int D = kHeadDim, NSTEP = 4, KB = TK / 16;
  constexpr bool UTILX = MODE == OBS_UTILX;
  constexpr bool HAS_V = MODE != OBS_STATS;
  constexpr bool HAS_G = MODE == OBS_UTIL || UTILX;   // anchor-dependent terms
  constexpr bool G_TILE = HAS_G && !QAT;               // gathered anchor rows in LDS
  static_assert(!QAT || MODE == OBS_UTIL, "anchor table only in the UTIL fast pass");
  extern __shared__ float qa_tab[];                    // QAT: [A16][GQp]
  constexpr bool HAS_PART = MODE != OBS_STATS;
  constexpr int TC = TK * 16;     // 16-byte chunks per [TK][128] bf16 tile
  constexpr float kLazy = 8.0f;   // STATS: rescale only when the max grows by more than 2^8
  using M = Mfma<ANCHORKV_BF16>;
  using frag = bf16x8;
  static_assert(TK == 32 || TK == 64, "32- or 64-key tiles");

  static_assert(ST >= 1 && ST <= 6 && (ST >= 2 || MODE == OBS_UTILX), "1..6 stages (1 only for UTILX)");
  // one distinct object per stage buffer: with a compile-time stage index the
  // compiler can tell compute reads from the copies in flight
#define AKV_STAGE_BUFS(j)                                                               \
  __shared__ __attribute__((aligned(16))) uint4 K##j[(ST > j) ? TC : 1];                \
  __shared__ __attribute__((aligned(16))) uint4 V##j[(HAS_V && ST > j) ? TC : 1];       \
  __shared__ __attribute__((aligned(16))) uint4 G##j[(G_TILE && ST > j) ? TC : 1];      \
  __shared__ __attribute__((aligned(16))) float S##j[(HAS_G && ST > j) ? 3 * kObsSlot : 1];
  AKV_STAGE_BUFS(0) AKV_STAGE_BUFS(1) AKV_STAGE_BUFS(2) AKV_STAGE_BUFS(3) AKV_STAGE_BUFS(4) AKV_STAGE_BUFS(5)
#undef AKV_STAGE_BUFS
  __shared__ int Ai[HAS_G ? kObsUtilMaxKeys : 1];   // anchor index of every key of the range
  __shared__ float part[HAS_PART ? 2 : 1][HAS_PART ? kObsMaxWaves : 1][kObsSlot];
  __shared__ float pflag[HAS_G ? 2 : 1][kObsSlot];
  __shared__ int tflag[MODE == OBS_UTIL ? 2 : 1][kObsMaxWaves * KS];

  static_assert(KS == 1 || (KS == 2 && MODE == OBS_UTIL), "key splits only in the UTIL fast pass");
  constexpr int KBW = KB / KS;   // 16-key blocks of a tile per wave
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;          // waves of the block (copies are spread over all)
  const int nq = nw / KS;                  // query-block waves per key split
  const int qw = wave % nq;                // this wave's query group
  const int kb0 = (wave / nq) * KBW;       // this wave's first 16-key block of a tile
  const int col = lane & 15, kg = lane >> 4;
  const int nsplit = HAS_G ? a.S1u : a.S1;
  const int kps = HAS_G ? a.kps_u : a.kps;
  int bid = blockIdx.x;
  const int s = bid % nsplit; bid /= nsplit;
  const int h = bid % a.H;
  const int u = bid / a.H;
  const int N = a.N, H = a.H;
  const int k0 = s * kps;
  const int k1 = min(N, k0 + kps);
  const int64_t uh = (int64_t)u * H + h;
  if (k0 >= k1) {
    // empty split: neutral partials
    if constexpr (MODE == OBS_STATS) {
      for (int qi = 0; qi < QPW; ++qi) {
        const int qb = wave + qi * nw;
        if (kg == 0 && qb * 16 < a.GQp) a.ml_part[(uh * a.S1 + s) * a.GQp + qb * 16 + col] = make_float2(-INFINITY, 0.0f);
      }
    }
    if constexpr (MODE == OBS_SCORE) {
      for (int qi = 0; qi < QPW; ++qi) {
        const int qb = wave + qi * nw;
        if (qb * 16 >= a.GQp) continue;
        for (int db = 0; db < 8; ++db)
          for (int r = 0; r < 4; ++r)
            a.o_part[((uh * a.S1 + s) * a.GQp + qb * 16 + kg * 4 + r) * D + db * 16 + col] = 0.0f;
      }
    }
    return;
  }
  const int ntiles = (k1 - k0 + TK - 1) / TK;
  uint8_t* fl = HAS_G ? a.uflag + uh * a.nflag + k0 / TK : nullptr;   // UTIL / UTILX tile flags of the range
  if constexpr (UTILX) {
    // nothing to redo in this range: leave before any other work
    bool any = false;
    for (int j = lane; j < ntiles; j += 64) any |= fl[j] != 0;
    if (__builtin_amdgcn_ballot_w64(any) == 0) return;
  }
  const uint16_t* Kp = reinterpret_cast<const uint16_t*>(a.K) + uh * N * D;
  const uint16_t* Vp = reinterpret_cast<const uint16_t*>(a.V) + uh * N * D;
  const uint16_t* Qp = reinterpret_cast<const uint16_t*>(a.Q) + ((int64_t)u * H * a.G + (int64_t)h * a.G) * a.n_obs * D;
  const uint16_t* Ap = reinterpret_cast<const uint16_t*>(a.cache + (int64_t)u * a.stride + a.off_anchor_k) +
                       (int64_t)h * a.A * D;
  const int64_t sideK = ((int64_t)u * 2 * H + h) * N;   // K-side rows of [U][2][H][N] arrays
  const DmaLane dl(lane);

  // ---- UTIL: anchor index of every key of the range, loaded once
  if constexpr (HAS_G) {
    for (int b = wave; b * 64 < k1 - k0; b += nw) {
      const int t = min(k0 + b * 64 + lane, k1 - 1);
      dma4(a.aidx + sideK + t, Ai + b * 64);
    }
  }

  // ---- per-wave query blocks (B fragments, constant over all keys)
  frag qf[QPW][NSTEP];
  frag ofh[HAS_G ? QPW : 1][NSTEP];
  frag ofl[HAS_G ? QPW : 1][NSTEP];
  float mqp[QPW];    // exponent offset: p = 2^(s c - mqp); +inf for padding queries
  float ooq[QPW];    // ||o||^2 of the lane's query
  int kmax[QPW];     // key t is visible to this lane's query iff t < kmax
  bool qactive[QPW];
  const int vis_base = N - a.n_obs;  // query j sees keys <= vis_base + j
  float oomax = 0.0f;
  for (int qi = 0; qi < QPW; ++qi) {
    const int qb = qw + qi * nq;
    const int q = qb * 16 + col;
    qactive[qi] = qb * 16 < a.GQp;
    const bool qvalid = qactive[qi] && q < a.GQ;
    kmax[qi] = qvalid ? min(k1, vis_base + q % a.n_obs + 1) : -1;
    for (int st = 0; st < NSTEP; ++st) {
      const int kk = st * 32 + kg * 8;
      qf[qi][st] = qvalid ? M::load(Qp + (int64_t)q * D + kk) : M::zero();
      if constexpr (HAS_G) {
        const uint16_t* oh = a.ohl + (uh * 2 + 0) * a.GQp * D;
        const uint16_t* ol = a.ohl + (uh * 2 + 1) * a.GQp * D;
        ofh[qi][st] = qvalid ? M::load(oh + (int64_t)q * D + kk) : M::zero();
        ofl[qi][st] = qvalid ? M::load(ol + (int64_t)q * D + kk) : M::zero();
      }
    }
    mqp[qi] = INFINITY;
    ooq[qi] = 0.0f;
    if constexpr (MODE != OBS_STATS) {
      if (qvalid) {
        const float2 v = a.ml[uh * a.GQp + q];   // (max logit * c, 1/l)
        mqp[qi] = v.x - log2f(v.y);
      }
    }
    if constexpr (HAS_G) {
      if (qvalid) ooq[qi] = a.oo[uh * a.GQp + q];
      oomax = fmaxf(oomax, ooq[qi]);
    }
  }
  // cancellation threshold offset of the wave (a quarter of the largest ||o||^2)
  const float oo4 = HAS_G ? 0.25f * wave_max(oomax) : 0.0f;
  // first key of the range that some query of the block must not see (or the range end)
  const int mask_from = min(k1, vis_base + 1);
  // STATS running max (log2 domain; finite start so that fully masked tiles
  // add exp2(-inf) = 0) and sum
  float m_run[QPW], l_run[QPW];
  for (int qi = 0; qi < QPW; ++qi) { m_run[qi] = -1e30f; l_run[qi] = 0.0f; }
  f32x4 oacc[MODE == OBS_SCORE ? QPW : 1][MODE == OBS_SCORE ? 8 : 1];
  if constexpr (MODE == OBS_SCORE)
    for (int qi = 0; qi < QPW; ++qi)
      for (int db = 0; db < 8; ++db) oacc[qi][db] = f32x4{0, 0, 0, 0};

  // ---- copies of tile `it` into buffers b
  // (returns the number of copy instructions this wave issued: the same for
  // every tile of the block)
  auto issue = [&](int it, const ObsBufs& b) -> int {
    const int t0 = k0 + it * TK;
    const int nval = min(TK, k1 - t0);
    int n = 0;
    if constexpr (HAS_G) {
      if constexpr (G_TILE) n += dma_gather<TK>(b.G, Ap, Ai + it * TK, nval, nw, wave, dl);
      const int tl = min(t0 + lane, k1 - 1);
      for (int arr = wave; arr < 3; arr += nw, ++n) {
        const void* src = arr == 0 ? (const void*)(a.gam + sideK + tl)
                        : arr == 1 ? (const void*)(a.vn2 + uh * N + tl)
                                   : (const void*)(a.anchor_of + uh * N + tl);
        dma4(src, b.S + arr * kObsSlot);
      }
    }
    n += dma_rows<TK>(b.K, Kp + (int64_t)t0 * D, nval, nw, wave, dl);
    if constexpr (HAS_V) n += dma_rows<TK>(b.V, Vp + (int64_t)t0 * D, nval, nw, wave, dl);
    return n;
  };
  // sum of the per-wave partials of tile `it` (one wave), fixed wave order
  auto combine = [&](int it) {
    if constexpr (HAS_PART) {
      if (wave == it % nw) {
        const int t = k0 + it * TK + lane;
        float v = 0.0f;
        for (int w = 0; w < nq; ++w) v += part[it & 1][w][lane];
        if (lane < TK && t < k1) {
          if constexpr (MODE == OBS_SCORE) {
            a.score[uh * N + t] = v;
          } else {
            a.util[sideK + t] = pflag[it & 1][lane] != 0.0f ? -1.0f : v * a.inv_sqrt_d;
          }
        }
        if constexpr (MODE == OBS_UTIL) {
          int any = 0;
          for (int w = 0; w < nw; ++w) any |= tflag[it & 1][w];
          if (lane == 0) fl[it] = any ? 1 : 0;
        }
      }
    }
  };
  // per-key sums over this wave's 16 query columns (DPP within rows of 16)
  // colsum[i] holds the 16-key block kbase + i
  auto write_part = [&](int it, const ObsBufs& c, auto& colsum, int kbase) {
    constexpr int NKB = sizeof(colsum) / sizeof(colsum[0]);
    float* pw = part[it & 1][qw];
    for (int i = 0; i < NKB; ++i) {
      const float v = row_sum4_scatter(colsum[i], col);
      if ((col & 3) == 0) pw[(kbase + i) * 16 + kg * 4 + (col >> 2)] = v;
    }
    if constexpr (HAS_G) {
      if (wave == 0) pflag[it & 1][lane] = reinterpret_cast<const int*>(c.S)[2 * kObsSlot + lane] >= 0 ? 1.0f : 0.0f;
    }
  };

  // ---- compute one tile from buffers c (MASK: apply the causal / range mask)
  auto compute = [&](auto maskc, int it, const ObsBufs& c) {
    constexpr bool MASK = decltype(maskc)::value;
    const int t0 = k0 + it * TK;
    float colsum[KBW][4];
    for (int kb = 0; kb < KBW; ++kb)
      for (int r = 0; r < 4; ++r) colsum[kb][r] = 0.0f;
    float xs[MODE == OBS_STATS ? QPW : 1][KB][4];   // STATS: logits of the tile
    float pv[MODE == OBS_SCORE ? QPW : 1][2][4];
    uint64_t cmask = 0;                             // UTIL: lanes whose ||v - o||^2 may cancel
    for (int kbi = 0; kbi < KBW; ++kbi) {
      const int kb = KS == 1 ? kbi : kb0 + kbi;
      frag af[NSTEP], gf[HAS_G ? NSTEP : 1], vf[HAS_G ? NSTEP : 1];
      const int row = kb * 16 + col;
      for (int st = 0; st < NSTEP; ++st) {
        af[st] = lds_frag(c.K, row, st * 4 + kg);
        if constexpr (HAS_G) {
          if constexpr (G_TILE) gf[st] = lds_frag(c.G, row, st * 4 + kg);
          vf[st] = lds_frag(c.V, row, st * 4 + kg);
        }
      }
      float gm[4], vv[4], thr[4];
      if constexpr (HAS_G) {
        const float4 gm4 = *reinterpret_cast<const float4*>(c.S + kb * 16 + kg * 4);
        const float4 vv4 = *reinterpret_cast<const float4*>(c.S + kObsSlot + kb * 16 + kg * 4);
        gm[0] = gm4.x; gm[1] = gm4.y; gm[2] = gm4.z; gm[3] = gm4.w;
        vv[0] = vv4.x; vv[1] = vv4.y; vv[2] = vv4.z; vv[3] = vv4.w;
        for (int r = 0; r < 4; ++r) thr[r] = fmaf(0.25f, vv[r], oo4);
      }
      for (int qi = 0; qi < QPW; ++qi) {
        if (qi > 0 && !qactive[qi]) continue;  // wave-uniform; block 0 is always active
        f32x4 acc = {0, 0, 0, 0}, accg = {0, 0, 0, 0};
        const float oinit = -0.5f * ooq[qi];
        f32x4 accv = {oinit, oinit, oinit, oinit};
        for (int st = 0; st < NSTEP; ++st) acc = M::mma(af[st], qf[qi][st], acc);
        if constexpr (HAS_G) {
          if constexpr (QAT) {
            const int qcol = (qw + qi * nq) * 16 + col;
            for (int r = 0; r < 4; ++r) accg[r] = qa_tab[__umul24(Ai[it * TK + kb * 16 + kg * 4 + r], a.GQp) + qcol];  // index < 2^15, GQp <= 256
          } else {
            for (int st = 0; st < NSTEP; ++st) accg = M::mma(gf[st], qf[qi][st], accg);
          }
          for (int st = 0; st < NSTEP; ++st) accv = M::mma(vf[st], ofh[qi][st], accv);
          for (int st = 0; st < NSTEP; ++st) accv = M::mma(vf[st], ofl[qi][st], accv);
        }
        for (int r = 0; r < 4; ++r) {
          const int t = t0 + kb * 16 + kg * 4 + r;
          if constexpr (MODE == OBS_STATS) {
            const float x = acc[r] * a.c;
            xs[qi][kb][r] = (!MASK || t < kmax[qi]) ? x : -INFINITY;
          } else {
            float p = exp2_fast(fmaf(acc[r], a.c, -mqp[qi]));
            if constexpr (MASK) p = t < kmax[qi] ? p : 0.0f;
            if constexpr (MODE == OBS_SCORE) {
              pv[qi][kb & 1][r] = p;
              colsum[kbi][r] += p;
            } else {
              // accv = <v, o> - ||o||^2 / 2, so ||v - o||^2 = ||v||^2 - 2 accv
              const float qr = fabsf(fmaf(-gm[r], accg[r], acc[r]));
              const float vo2 = fmaf(-2.0f, accv[r], vv[r]);
              cmask |= __builtin_amdgcn_ballot_w64(vo2 < thr[r]);
              colsum[kbi][r] = fmaf(p * qr, __builtin_amdgcn_sqrtf(vo2), colsum[kbi][r]);
            }
          }
        }
      }
      if constexpr (MODE == OBS_SCORE) {
        if (kb & 1) {
          // P V for the 32-key chunk c2 = kb/2: value B fragments by transposing reads
          const int c2 = kb >> 1;
          const int g = lane >> 4, m = lane & 15;
          frag vb[8];
          for (int db = 0; db < 8; ++db) {
            const int d = db * 16 + (m & 3) * 4;
            const uint2 lo = lds_tr(c.V, c2 * 32 + g * 4 + (m >> 2), d);
            const uint2 hi = lds_tr(c.V, c2 * 32 + 16 + g * 4 + (m >> 2), d);
            vb[db] = bits_to_frag(make_uint4(lo.x, lo.y, hi.x, hi.y));
          }
          for (int qi = 0; qi < QPW; ++qi) {
            if (qi > 0 && !qactive[qi]) continue;
            float p8[8];
            for (int e = 0; e < 8; ++e) p8[e] = pv[qi][e >> 2][e & 3];
            bf16x8 ph, pl;
            split8(p8, ph, pl);
            for (int db = 0; db < 8; ++db) {
              oacc[qi][db] = M::mma(ph, vb[db], oacc[qi][db]);
              oacc[qi][db] = M::mma(pl, vb[db], oacc[qi][db]);
            }
          }
        }
      }
    }
    if constexpr (MODE == OBS_STATS) {
      // online softmax statistics, one (lazy) rescale per tile
      for (int qi = 0; qi < QPW; ++qi) {
        if (qi > 0 && !qactive[qi]) continue;
        float tmax = xs[qi][0][0];
        for (int kb = 0; kb < KB; ++kb)
          for (int r = 0; r < 4; ++r) tmax = fmaxf(tmax, xs[qi][kb][r]);
        if (tmax > m_run[qi] + kLazy) {
          l_run[qi] *= exp2_fast(m_run[qi] - tmax);
          m_run[qi] = tmax;
        }
        float l = l_run[qi];
        for (int kb = 0; kb < KB; ++kb)
          for (int r = 0; r < 4; ++r) l += exp2_fast(xs[qi][kb][r] - m_run[qi]);
        l_run[qi] = l;
      }
    }
    if constexpr (HAS_PART) write_part(it, c, colsum, KS == 1 ? 0 : kb0);
    if constexpr (MODE == OBS_UTIL) {
      if (lane == 0) tflag[it & 1][wave] = cmask != 0;
    }
  };

  // ---- UTILX: one flagged tile, with ||v - o||^2 evaluated directly where
  // the expanded form falls below half of ||v||^2 + ||o||^2
  auto compute_exact = [&](int it, const ObsBufs& c) {
    const int t0 = k0 + it * TK;
    float colsum[KB][4];
    for (int kb = 0; kb < KB; ++kb)
      for (int r = 0; r < 4; ++r) colsum[kb][r] = 0.0f;
    for (int kb = 0; kb < KB; ++kb) {
      frag af[NSTEP], gf[NSTEP], vf[NSTEP];
      const int row = kb * 16 + col;
      for (int st = 0; st < NSTEP; ++st) {
        af[st] = lds_frag(c.K, row, st * 4 + kg);
        gf[st] = lds_frag(c.G, row, st * 4 + kg);
        vf[st] = lds_frag(c.V, row, st * 4 + kg);
      }
      for (int qi = 0; qi < QPW; ++qi) {
        if (qi > 0 && !qactive[qi]) continue;
        f32x4 acc = {0, 0, 0, 0}, accg = {0, 0, 0, 0}, accv = {0, 0, 0, 0};
        for (int st = 0; st < NSTEP; ++st) acc = M::mma(af[st], qf[qi][st], acc);
        for (int st = 0; st < NSTEP; ++st) accg = M::mma(gf[st], qf[qi][st], accg);
        for (int st = 0; st < NSTEP; ++st) accv = M::mma(vf[st], ofh[qi][st], accv);
        for (int st = 0; st < NSTEP; ++st) accv = M::mma(vf[st], ofl[qi][st], accv);
        for (int r = 0; r < 4; ++r) {
          const int kl = kb * 16 + kg * 4 + r;
          if (t0 + kl >= kmax[qi]) continue;
          const float p = exp2_fast(fmaf(acc[r], a.c, -mqp[qi]));
          if (!(p > 0.0f)) continue;
          const float gm = c.S[kl], vv = c.S[kObsSlot + kl];
          const float qr = fabsf(fmaf(-gm, accg[r], acc[r]));
          const float sum = vv + ooq[qi];
          float vo2 = fmaf(-2.0f, accv[r], sum);
          if (vo2 < 0.5f * sum) {
            const int q = (qw + qi * nq) * 16 + col;
            const float* orow = a.ofull + (uh * a.GQp + q) * D;
            const uint16_t* vrow = reinterpret_cast<const uint16_t*>(c.V);
            float acc2 = 0.0f;
            for (int d = 0; d < D; ++d) {
              const float df = bf2f(vrow[obs_phys(kl, d >> 3) * 8 + (d & 7)]) - orow[d];
              acc2 = fmaf(df, df, acc2);
            }
            vo2 = acc2;
          }
          colsum[kb][r] = fmaf(p * qr, __builtin_amdgcn_sqrtf(fmaxf(vo2, 0.0f)), colsum[kb][r]);
        }
      }
    }
    write_part(it, c, colsum, 0);
  };

  const ObsBufs B[6] = {{K0, V0, G0, S0}, {K1, V1, G1, S1}, {K2, V2, G2, S2},
                        {K3, V3, G3, S3}, {K4, V4, G4, S4}, {K5, V5, G5, S5}};
  if constexpr (HAS_G) {
    wait_vm_all();     // anchor indices before the gathers that use them
    __syncthreads();
  }
  if constexpr (QAT) {
    // table rows of 16 anchors per MFMA (A operand: anchor rows from the
    // cache; B: this wave's query fragments); the key splits share the blocks
    const int nab = (a.A + 15) / 16;
    for (int qi = 0; qi < QPW; ++qi) {
      if (qi > 0 && !qactive[qi]) continue;
      const int qcol = (qw + qi * nq) * 16 + col;
      for (int ab = wave / nq; ab < nab; ab += KS) {
        const int arow = min(ab * 16 + col, a.A - 1);
        f32x4 acc = {0, 0, 0, 0};
        for (int st = 0; st < NSTEP; ++st) acc = M::mma(M::load(Ap + (int64_t)arow * D + st * 32 + kg * 8), qf[qi][st], acc);
        for (int r = 0; r < 4; ++r) qa_tab[(ab * 16 + kg * 4 + r) * a.GQp + qcol] = acc[r];
      }
    }
    __syncthreads();
  }
  if constexpr (UTILX) {
    for (int it = 0; it < ntiles; ++it) {
      if (__builtin_amdgcn_readfirstlane((int)fl[it]) == 0) continue;
      issue(it, B[0]);
      wait_vm_all();
      __syncthreads();
      compute_exact(it, B[0]);
      __syncthreads();
      combine(it);
      __syncthreads();
    }
    return;
  } else {
    // ---- prologue: tiles 0 .. ST-2 in flight
    int nper = 0;   // copy instructions per tile (this wave)
#pragma unroll
    for (int j = 0; j < ST - 1; ++j)
      if (j < ntiles) nper = issue(j, B[j]);
    wait_vm_le(nper * (min(ST - 1, ntiles) - 1));   // tile 0 has landed
    // ---- one step: tile `it` from buffers c while tile it+ST-1 is copied into buffers n
    auto step = [&](int it, const ObsBufs& c, const ObsBufs& n) {
      // LDS-only barrier: a full __syncthreads would also wait for the
      // copies still in flight
      lds_barrier();
      if (it > 0) combine(it - 1);
      if (it + ST - 1 < ntiles) issue(it + ST - 1, n);
      if (k0 + (it + 1) * TK > mask_from) compute(std::true_type{}, it, c);
      else compute(std::false_type{}, it, c);
      // tile it+1 has landed (this wave's copies; the next barrier covers the
      // others); the copies of tiles it+2 .. it+ST-1 may stay in flight
      wait_vm_le(nper * max(0, min(it + ST - 1, ntiles - 1) - (it + 1)));
    };
    for (int it0 = 0; it0 < ntiles; it0 += ST) {
#pragma unroll
      for (int j = 0; j < ST; ++j)
        if (it0 + j < ntiles) step(it0 + j, B[j], B[(j + ST - 1) % ST]);
    }
    __syncthreads();
    combine(ntiles - 1);
  }

  if constexpr (MODE == OBS_STATS) {
    for (int qi = 0; qi < QPW; ++qi) {
      float m = l_run[qi] > 0.0f ? m_run[qi] : -INFINITY, l = l_run[qi];
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
