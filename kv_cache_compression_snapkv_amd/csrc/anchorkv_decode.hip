// Decode attention over the compressed cache (gfx950).
//
// For q-head g of KV head h (Pith review of AnchorKV, "What carries the
// argument": x^_t = gamma_t x_a(t) + r~_t):
//   logit_t = gamma^K_t <q, k_a> / sqrt(D) + [t in R_K] <q, r~^K_t> / sqrt(D)
//   o = sum_t p_t (gamma^V_t v_a(t) + [t in R_V] r~^V_t) / sum_t p_t
// computed without reconstructing K or V (the paper's fused-decoder idea,
// AnchorKV-adapted page "Adaptation notes"; the design here is our own), in
// one kernel:
//  * prologue: the anchor logits S[a][g] = <q_g, k_a> log2(e)/sqrt(D) on MFMA
//    into LDS;
//  * tiles of 1024 tokens: S lookups, residual-key logits, softmax weights;
//    the value side scatters p_t gamma^V_t into w[a(t)][g] (LDS, 64-bit fixed
//    point with scale 2^38, each term rounded to nearest: LDS integer atomics
//    are an order of magnitude faster than LDS float atomics on this part and
//    make the sum independent of order) and sums p r~^V on MFMA;
//  * epilogue: w V_anchors on MFMA plus the residual part; with several
//    token ranges per head, the last range's workgroup merges the partial
//    (max, sum, output) triples.
// Residual records are handled in batches on MFMA.  A code c enters as an
// exact bf16 value 128 + c * 4^m (one AND-OR per pair of codes) and the
// constant part is cancelled exactly.  Keys: rows = records, columns =
// (q-head, group), so one 16x16 tile serves 4 q-heads x 4 groups.  Values:
// rows = (q-head, group), K = records, columns = coordinates; A = p * scale
// split into bf16 hi + lo.
// One workgroup (8 waves) per (unit, head, 1024-token-aligned range).  The
// running max is shared by the workgroup and only raised (rescaling w, l and
// the accumulators) when a tile exceeds it by more than 2^1, so p <= 2.
//
// Fixed-point range: a term is p gamma 2^38 rounded to the nearest integer,
// so terms down to about 2^-28 of the running maximum keep 10 significant
// bits and the rounding bias over a whole range (<= 2^17 tokens) stays below
// 2^-21 of it; a peaked softmax (a few keys 15-20 nats above a long flat
// background) therefore keeps its background mass.  The sum over a range
// stays below 2^63 while the mean |gamma| of its tokens is below 2^6.
#include "device_common.hpp"
#include "launch_common.hpp"

#include <algorithm>
#include <type_traits>

namespace akv {


constexpr int kMaxG = 8;          // q-heads per KV head supported by decode
constexpr int kTile = 1024;       // tokens per tile (= residual-offset chunk)
constexpr int kWaves = 8;         // waves per workgroup; 128 tokens per wave per tile
constexpr uint32_t kCodeBias = 0x43004300u;  // bf16 pair (128, 128)
constexpr float kFxScale = 0x1p38f;               // fixed-point scale of the w scatter
constexpr double kFxScaleD = 0x1p38;
constexpr double kFxInv = 0x1p-38;
constexpr double kRoundMagic = 0x1.8p52;           // x + 1.5*2^52 rounds x (|x| < 2^51) to an integer
constexpr unsigned long long kMagicMask = 0x0007FFFFFFFFFFFFull;  // low 51 bits: that integer, for x >= 0
constexpr float kLazy = 1.0f;                      // rescale when a logit passes m_run + kLazy (log2 units)
// floats of the per-tile buffer: [kTile][G], at least the 8 KB of staged words
template <int G> constexpr int kBufFloats = kTile * G > 2048 ? kTile * G : 2048;

// y (already scaled by 2^38) -> two's-complement 64-bit fixed point, any sign
// and |y| < 2^62.
__device__ __forceinline__ unsigned long long fx_general(float y) {
  const float a = fabsf(y);
  const float hi_f = floorf(a * 2.3283064365386963e-10f);  // 2^-32
  const float lo_f = fmaf(hi_f, -4294967296.0f, a);           // exact, in [0, 2^32)
  const unsigned long long v = ((unsigned long long)(unsigned)hi_f << 32) | (unsigned long long)(unsigned)rintf(lo_f);
  return y < 0.0f ? 0ull - v : v;
}

// ---------------------------------------------------------------- stream
struct DecArgs {
  const void* q;
  const uint8_t* cache;
  int64_t stride, off_words, off_rk, off_rv, off_ck, off_cv, off_ak, off_av;
  float2* part_ml;   // [U][H][S2][G] (max, sum) of each range (S2 > 1 or a tail follows)
  float* part_acc;   // [U][H][S2][G][D] unnormalised output of each range (same cases)
  float* o;          // [U][H][G][D]
  int H, N, A, C, S2, cps, R_K, R_V;
  int force_part;    // publish partials even with one range (a tail follows)
  float c;
};

// Record staging: KP 16-byte chunks per thread per side are prefetched, so a
// tile stages up to 512*KP*16/48 records per side in LDS; records beyond that
// are read from the cache directly.

__device__ __forceinline__ bf16x8 u4_to_frag(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return bits_to_frag(make_uint4(a, b, c, d));
}

// (a & m) | b: with m an opaque SGPR value and b an opaque VGPR value (see
// the kernel prologue) the compiler selects one v_and_or_b32; with both as
// literals it would split it (the three-operand encoding takes no literal
// here).  Plain C on purpose: an instruction hidden in inline asm is invisible
// to the compiler's hazard checks, which must order it against MFMA writes.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t b) { return (a & m) | b; }

typedef __attribute__((ext_vector_type(2))) float f32x2v;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2v;
// two floats -> packed bf16 pair (round to nearest even), lo in bits 0..15
__device__ __forceinline__ uint32_t bf16_pack(float lo, float hi) {
  const f32x2v f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2v));
}

// Code planes.  In a record, code word j holds coordinates j + 16c (c = 0..7)
// at bits p = 2c, p + 1.  A 32-bit word of two code words, shifted right by
// sh in {0, 6, 12}, has the field of plane c at bits 2m, 2m + 1 (m = 0, 1, 2)
// of both halves; masking it there and OR-ing the exponent of 128 gives the
// exact bf16 pair 128 + code * 4^m.  The 4^m is folded into the other MFMA
// operand (keys) or removed at the end (values); the 128 is cancelled by the
// accumulator's initial value (keys) or by a bias MFMA (values).
struct Plane {
  int sh, m;
};
__device__ constexpr Plane plane_of(int c) {
  return c < 3 ? Plane{0, c} : c < 6 ? Plane{6, c - 3} : Plane{12, c - 6};
}
constexpr float kPlaneInv[3] = {1.0f, 0.25f, 0.0625f};

// ordered-int image of a float (monotone), for LDS integer max
__device__ __forceinline__ int fkey(float f) {
  const int b = __float_as_int(f);
  return b >= 0 ? b : b ^ 0x7FFFFFFF;
}
__device__ __forceinline__ float fkey_inv(int k) { return __int_as_float(k >= 0 ? k : k ^ 0x7FFFFFFF); }
constexpr int kKeyNegInf = (int)0x807FFFFF;  // fkey(-inf)

template <int N> struct FVec;
template <> struct FVec<1> { using T = float; };
template <> struct FVec<2> { using T = float2; };
template <> struct FVec<4> { using T = float4; };
// GP consecutive floats from / to LDS (16-byte aligned for GP >= 4)
template <int GP> __device__ __forceinline__ void ldsv(const float* p, float (&o)[GP]) {
  if constexpr (GP <= 4) {
    const typename FVec<GP>::T v = *reinterpret_cast<const typename FVec<GP>::T*>(p);
    __builtin_memcpy(o, &v, sizeof(v));
  } else {
#pragma unroll
    for (int k = 0; k < GP / 4; ++k) {
      const float4 v = reinterpret_cast<const float4*>(p)[k];
      o[4 * k] = v.x; o[4 * k + 1] = v.y; o[4 * k + 2] = v.z; o[4 * k + 3] = v.w;
    }
  }
}
template <int GP> __device__ __forceinline__ void stsv(float* p, const float (&o)[GP]) {
  if constexpr (GP <= 4) {
    typename FVec<GP>::T v;
    __builtin_memcpy(&v, o, sizeof(v));
    *reinterpret_cast<typename FVec<GP>::T*>(p) = v;
  } else {
#pragma unroll
    for (int k = 0; k < GP / 4; ++k)
      reinterpret_cast<float4*>(p)[k] = make_float4(o[4 * k], o[4 * k + 1], o[4 * k + 2], o[4 * k + 3]);
  }
}

// MFMA operand from KW consecutive floats in LDS (bf16: 8, exact for bf16
// data; f32: 1); zeros when !valid
template <int DT> __device__ __forceinline__ typename Mfma<DT>::frag frag_of(const float* p, bool valid) {
  if constexpr (DT == ANCHORKV_BF16) {
    if (!valid) return Mfma<DT>::zero();
    const float4 x = reinterpret_cast<const float4*>(p)[0], y = reinterpret_cast<const float4*>(p)[1];
    return u4_to_frag(bf16_pack(x.x, x.y), bf16_pack(x.z, x.w), bf16_pack(y.x, y.y), bf16_pack(y.z, y.w));
  } else {
    return valid ? *p : 0.0f;
  }
}

// set bits of a wave mask below this lane
__device__ __forceinline__ int lanes_below(unsigned long long m) {
  return (int)__builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
}

template <int G> constexpr int kGPad = G <= 1 ? 1 : G <= 2 ? 2 : G <= 4 ? 4 : 8;
constexpr int kRecPad = 32;  // zeroed records after the value staging (batch tails read them)

template <int DT, int G, int KP, int DEPTH, int WPE>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(WPE))) void k_dec_stream(DecArgs a) {
  constexpr int kPre = KP;
  constexpr int kRecCap = 512 * KP * 16 / kRecBytes;
  using T = typename Elem<DT>::T;
  using M = Mfma<ANCHORKV_BF16>;
  constexpr int D = kHeadDim;
  constexpr int GP = kGPad<G>;                   // q-heads per anchor row in LDS (padded)
  constexpr int NB = (4 * G + 15) / 16;          // 16-wide blocks of (q-head, group) pairs
  constexpr bool QSPLIT = DT == ANCHORKV_F32;   // f32 queries enter the key MFMA as bf16 hi + lo
  extern __shared__ __align__(16) float sm[];
  const int A = a.A;
  // w[g][a] in fixed point, q-head-major: the scatter's random anchors then
  // spread over all banks (an anchor-major row of GP entries would put every
  // anchor's entry g on the same few banks)
  unsigned long long* wi = reinterpret_cast<unsigned long long*>(sm);  // [GP][A]
  float* S = reinterpret_cast<float*>(wi + A * GP);                      // [A][GP]
  // [kTile][BR]: per wave 128 private rows (its tokens' records by rank):
  // key-residual logits, then p of value-flagged tokens (zeros in columns
  // >= G and in the rows up to the next 32); [G][D] at the end.  At the start
  // of a tile it first holds the staged pointer words ([512] x 16 B).
  constexpr int BR = 4 * NB;
  float* buf = sm + ((3 * GP * A + 3) & ~3);
  uint4* wst = reinterpret_cast<uint4*>(buf);
  uint4* kst = reinterpret_cast<uint4*>(buf + kBufFloats<BR>);  // staged key records of the tile
  uint4* vst = kst + 512 * kPre;                                 // staged value records, then kRecPad zero records
  const uint8_t* kstb = reinterpret_cast<const uint8_t*>(kst);
  const uint8_t* vstb = reinterpret_cast<const uint8_t*>(vst);
  __shared__ int cnt[kWaves];  // per wave: key-flagged | value-flagged << 16
  __shared__ int offs[2][130];
  __shared__ __align__(16) int tmaxb[2][GP];
  __shared__ __align__(16) float zrow[GP];
  __shared__ float zt_s[G * 4];

  int bid = blockIdx.x;
  const int sp = bid % a.S2; bid /= a.S2;
  const int h = bid % a.H;
  const int u = bid / a.H;
  const int64_t uh = (int64_t)u * a.H + h;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave: uniform
  const int col = lane & 15, kg = lane >> 4;
  float* wbuf = buf + wave * 128 * BR;  // this wave's rows
  const int c0 = sp * a.cps, c1 = min(a.C, c0 + a.cps);
  const int t_beg = c0 * kTile, t_end = min(a.N, c1 * kTile);
  const uint8_t* base = a.cache + (int64_t)u * a.stride;
  const uint8_t* recK = base + a.off_rk;
  const uint8_t* recV = base + a.off_rv;
  const T* q = reinterpret_cast<const T*>(a.q) + uh * G * D;

  // The unit's header must describe the cache the plan describes; a unit that
  // does not (another plan's cache, a unit never written) gives NaN outputs
  // and nothing past its header is read.  Uniform: every thread reads the
  // same words.
  {
    const UnitHeader* hd = reinterpret_cast<const UnitHeader*>(base);
    if (hd->magic != kMagic || hd->H != a.H || hd->N != a.N || hd->A != A || hd->R_K != a.R_K || hd->R_V != a.R_V ||
        hd->unit_stride != a.stride || hd->off_words != a.off_words) {
      const float nan = __builtin_nanf("");
      if (a.S2 == 1 && !a.force_part) {
        for (int i = threadIdx.x; i < G * D; i += blockDim.x) a.o[uh * G * D + i] = nan;
      } else {
        const int64_t ps = uh * a.S2 + sp;
        for (int i = threadIdx.x; i < G * D; i += blockDim.x) a.part_acc[ps * G * D + i] = nan;
        if (threadIdx.x < G) a.part_ml[ps * G + threadIdx.x] = make_float2(nan, nan);
      }
      return;
    }
  }

  // q of this head as floats in LDS ([G][D]; buf is free until the first tile)
  float* qf = buf;
  for (int i = threadIdx.x; i < G * D; i += blockDim.x) qf[i] = Elem<DT>::f(q[i]);
  for (int i = threadIdx.x; i < GP * A; i += blockDim.x) wi[i] = 0ull;
  for (int i = threadIdx.x; i < kRecPad * kRecBytes / 16; i += blockDim.x) vst[512 * kPre + i] = make_uint4(0, 0, 0, 0);
  if (threadIdx.x < G * 4) zt_s[threadIdx.x] = 0.0f;
  if (threadIdx.x < GP) {
    zrow[threadIdx.x] = 0.0f;
    tmaxb[0][threadIdx.x] = kKeyNegInf;
    tmaxb[1][threadIdx.x] = kKeyNegInf;
  }
  // record offsets of the range's chunks and of the chunk after the last one
  const int nch = max(0, c1 - c0);
  for (int i = threadIdx.x; i <= nch; i += blockDim.x) {
    const int fl = h * a.C + c0 + i;
    const bool last = fl >= a.H * a.C;
    offs[0][i] = last ? a.R_K : reinterpret_cast<const int*>(base + a.off_ck)[fl];
    offs[1][i] = last ? a.R_V : reinterpret_cast<const int*>(base + a.off_cv)[fl];
  }
  __syncthreads();  // qf, offs

  // code-plane constants: masks (SGPRs) and the exponent bias (one VGPR)
  uint32_t MK[3] = {0x00030003u, 0x000C000Cu, 0x00300030u};
  asm volatile("" : "+s"(MK[0]), "+s"(MK[1]), "+s"(MK[2]));
  uint32_t vbias = kCodeBias;
  asm volatile("" : "+v"(vbias));

  // Key-side B fragments: column kappa = 16*cb + col = 4*g + grp; in MFMA step
  // st (= coordinate group st) the lane supplies q[g][d] / 4^m for
  // d = j + 16c, j = 4kg + (e&3), c = 2st + (e>>2), when grp == st, zeros
  // otherwise.  cinit = -128 * (sum of what the column is fed), so the
  // accumulator ends at sum_d q[g][d] * code_d.
  // the fragments are the same in every wave: kept in LDS (after the value
  // staging and its zero records), written by wave 0
  constexpr int QH = QSPLIT ? 2 : 1;
  uint4 (*qbs)[64] = reinterpret_cast<uint4 (*)[64]>(vst + 512 * kPre + kRecPad * kRecBytes / 16);
  // per lane (column): sum of q over the column's group and cinit, also in
  // LDS (after the fragments) so that they take no registers in the tile loop
  float2* qcs = reinterpret_cast<float2*>(qbs + NB * 4 * QH);  // [NB][64]
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) {
    const int kap = 16 * cb + col;
    const int g = kap >> 2, grp = kap & 3;
    float qs = 0.0f, fed = 0.0f;
    if (g < G)
      for (int d = 32 * grp; d < 32 * grp + 32; ++d) {
        const float x = qf[g * D + d];
        const float sc = kPlaneInv[plane_of(d >> 4).m];
        const float xh = bf2f(f2bf(x));
        qs += x;
        fed += xh * sc;
        if constexpr (QSPLIT) fed += bf2f(f2bf(x - xh)) * sc;
      }
    if (wave == 0) qcs[cb * 64 + lane] = make_float2(qs, -128.0f * fed);
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      uint16_t vh[8], vl[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = 2 * st + (e >> 2);
        const int d = (4 * kg + (e & 3)) + 16 * c;
        const float x = (g < G && grp == st) ? qf[g * D + d] : 0.0f;
        const float sc = kPlaneInv[plane_of(c).m];
        vh[e] = f2bf(x);
        vl[e] = f2bf(x - bf2f(vh[e]));
        vh[e] = f2bf(bf2f(vh[e]) * sc);  // exact: power-of-two scaling
        vl[e] = f2bf(bf2f(vl[e]) * sc);
      }
      if (wave == 0) {
        qbs[(cb * 4 + st) * QH][lane] = make_uint4(vh[0] | (uint32_t)vh[1] << 16, vh[2] | (uint32_t)vh[3] << 16,
                                                   vh[4] | (uint32_t)vh[5] << 16, vh[6] | (uint32_t)vh[7] << 16);
        if constexpr (QSPLIT)
          qbs[(cb * 4 + st) * QH + 1][lane] = make_uint4(vl[0] | (uint32_t)vl[1] << 16, vl[2] | (uint32_t)vl[3] << 16,
                                                         vl[4] | (uint32_t)vl[5] << 16, vl[6] | (uint32_t)vl[7] << 16);
      }
    }
  }
  // value side: B = -128 everywhere cancels the code bias of the A rows
  const bf16x8 bm128 = u4_to_frag(0xC300C300u, 0xC300C300u, 0xC300C300u, 0xC300C300u);

  float m_run[G], lacc[G];
#pragma unroll
  for (int g = 0; g < G; ++g) { m_run[g] = -INFINITY; lacc[g] = 0.0f; }
  // value side, row block rb (rows 4g + grp), column block cc (coordinates
  // j + 16cc): of each MFMA tile only the rows of group cc/2 are wanted, so a
  // batch's tile starts from the batch's code-bias term -128 * (row sums of
  // A) and its row r = cc/2 is added to vacc (scaled by 4^m of the plane)
  float vacc[NB][8];
#pragma unroll
  for (int rb = 0; rb < NB; ++rb)
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) vacc[rb][cc] = 0.0f;
  float zt[NB];        // value side: sum of p * zero for row (rb, col)
#pragma unroll
  for (int rb = 0; rb < NB; ++rb) zt[rb] = 0.0f;

  const uint32_t* words = reinterpret_cast<const uint32_t*>(base + a.off_words) + (int64_t)h * a.N * 2;

  // Prefetch (registers), DEPTH tiles ahead: the thread's two pointer-word
  // pairs (one 16-byte load) and its share of the tile's key / value record
  // bytes (16-byte chunks).  The tile loop is unrolled by DEPTH so ring slots
  // stay static; each slot is emptied into LDS before it is reloaded.
  uint4 pw[DEPTH];
  uint4 pk[DEPTH][kPre], pv_[DEPTH][kPre];
  // All loads go through range-checked buffer resources: a lane past the
  // range (or a tile past the last) reads zeros and no memory.  For an odd
  // last token the range is rounded up to 16 bytes: the 8 bytes after this
  // head's words (the next head's or the chunk table) lie inside the unit and
  // the token-validity flags below ignore them.
  const __amdgpu_buffer_rsrc_t wrs = buf_rsrc(words + (int64_t)t_beg * 2, (uint32_t)(((t_end - t_beg) * 8 + 15) & ~15));
  auto prefetch = [&](int i, uint4& w_, uint4* k_, uint4* v_) {
    w_ = buf_load16(wrs, (uint32_t)(i * kTile + wave * 128 + 2 * lane) * 8u);
    const int ic = max(0, min(i, nch - 1));
    const int ok0 = __builtin_amdgcn_readfirstlane(offs[0][ic]), ok1 = __builtin_amdgcn_readfirstlane(offs[0][ic + 1]);
    const int ov0 = __builtin_amdgcn_readfirstlane(offs[1][ic]), ov1 = __builtin_amdgcn_readfirstlane(offs[1][ic + 1]);
    const int nk = i < nch ? 3 * min(kRecCap, ok1 - ok0) : 0;
    const int nv = i < nch ? 3 * min(kRecCap, ov1 - ov0) : 0;
    const __amdgpu_buffer_rsrc_t krs = buf_rsrc(recK + (int64_t)ok0 * kRecBytes, (uint32_t)nk * 16u);
    const __amdgpu_buffer_rsrc_t vrs = buf_rsrc(recV + (int64_t)ov0 * kRecBytes, (uint32_t)nv * 16u);
#pragma unroll
    for (int k = 0; k < kPre; ++k) {
      const uint32_t ci = threadIdx.x + 512 * k;
      k_[k] = buf_load16(krs, ci * 16u);
      v_[k] = buf_load16(vrs, ci * 16u);
    }
  };
  // issue order = slot order (the loop's waits count the loads issued after a
  // slot's, so the scheduler must not interleave the slots here)
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) {
    prefetch(d, pw[d], pk[d], pv_[d]);
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- anchor logits S[a][g] = <q_g, k_a> * c on MFMA, 16 anchors per tile
  // (rows = anchors, K = coordinates, columns = q-heads), while the first
  // tiles' loads are in flight
  {
    using MS = Mfma<DT>;
    const T* AK = reinterpret_cast<const T*>(base + a.off_ak) + (int64_t)h * A * D;
#pragma unroll 2
    for (int t = wave; t < (A + 15) / 16; t += kWaves) {
      const int ar = 16 * t + col;
      f32x4 sacc = {0, 0, 0, 0};
#pragma unroll
      for (int k0 = 0; k0 < D; k0 += MS::KSTEP) {
        const int kk = k0 + kg * MS::KW;
        const typename MS::frag af = ar < A ? MS::load(AK + (int64_t)ar * D + kk) : MS::zero();
        sacc = MS::mma(af, frag_of<DT>(qf + col * D + kk, col < G), sacc);
      }
      if (col < G)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int aa = 16 * t + 4 * kg + r;
          if (aa < A) S[aa * GP + col] = sacc[r] * a.c;
        }
    }
  }
  __syncthreads();  // S, qbs; qf is dead (buf becomes the tiles' buffer)

  for (int base_it = 0; base_it < nch; base_it += DEPTH) {
#pragma unroll
  for (int dslot = 0; dslot < DEPTH; ++dslot) {
    // no early exit: a tile past the range (odd tile count) reads nothing and
    // contributes nothing, and a branch out of the middle of the unrolled body
    // would let the compiler's wait counting assume a path that skipped the
    // other slot's loads
    const int it = base_it + dslot;
    const int par = it & 1;
    const int tile = t_beg + it * kTile;
    const int rk0 = offs[0][min(it, nch)], rv0 = offs[1][min(it, nch)];
    // stage this tile's records (the previous tile ended with a barrier)
#pragma unroll
    for (int k = 0; k < kPre; ++k) { kst[threadIdx.x + 512 * k] = pk[dslot][k]; vst[threadIdx.x + 512 * k] = pv_[dslot][k]; }
    wst[threadIdx.x] = pw[dslot];
    // compiler-only fence: the words are read back from LDS below instead of
    // being forwarded from pw, whose registers are free now for the next
    // prefetch
    asm volatile("" ::: "memory");
    prefetch(it + DEPTH, pw[dslot], pk[dslot], pv_[dslot]);
    const uint4 w4 = wst[threadIdx.x];  // own write, no barrier needed
    // ---- A: pointer words of the lane's two tokens
    const int t0 = tile + wave * 128 + 2 * lane;
    const bool v0 = t0 < t_end, v1 = t0 + 1 < t_end;
    const int aK0 = w4.x & 0x7FFF, aV0 = w4.y & 0x7FFF, aK1 = w4.z & 0x7FFF, aV1 = w4.w & 0x7FFF;
    // a token past the range has all-zero words (flags clear) except the odd
    // one after the last token, masked by v1
    const bool fK0 = w4.x & 0x8000u, fV0 = w4.y & 0x8000u;
    const bool fK1 = v1 && (w4.z & 0x8000u), fV1 = v1 && (w4.w & 0x8000u);
    const float gK0 = h2f((uint16_t)(w4.x >> 16)), gV0 = h2f((uint16_t)(w4.y >> 16));
    const float gK1 = h2f((uint16_t)(w4.z >> 16)), gV1 = h2f((uint16_t)(w4.w >> 16));
    const unsigned long long bK0 = __ballot(fK0), bK1 = __ballot(fK1), bV0 = __ballot(fV0), bV1 = __ballot(fV1);
    const int nK = __popcll(bK0) + __popcll(bK1), nV = __popcll(bV0) + __popcll(bV1);
    if (lane == 0) cnt[wave] = nK | (nV << 16);
    if (threadIdx.x < GP) tmaxb[par ^ 1][threadIdx.x] = kKeyNegInf;  // next tile's max (last read a tile ago)
    lds_barrier();
    // counts of the earlier waves: lanes 0..wave-1 hold them, summed over the row
    const int pre = __builtin_amdgcn_readfirstlane(row_sum_i32(lane < wave ? cnt[lane & (kWaves - 1)] : 0));
    const int baseK = pre & 0xFFFF, baseV = pre >> 16;
    // ranks of the lane's tokens among this wave's flagged ones
    const int rK0 = lanes_below(bK0) + lanes_below(bK1), rK1 = rK0 + (fK0 ? 1 : 0);
    const int rV0 = lanes_below(bV0) + lanes_below(bV1), rV1 = rV0 + (fV0 ? 1 : 0);

    // ---- B: key-residual logits of this wave's records, 16 per MFMA tile,
    // into this wave's buf rows [0, nK).  Batches
    // whose records are all staged read LDS only; the rest (tiles with more
    // flagged tokens than the staging holds) read the cache directly.
    auto kbatch = [&](int b0, auto from_lds) {
      constexpr bool LDS = decltype(from_lds)::value;
      const int i = b0 + col;
      uint2 x = make_uint2(0, 0);
      if constexpr (LDS) x = *reinterpret_cast<const uint2*>(kstb + (baseK + i) * kRecBytes + 8 * kg);
      else if (i < nK) x = *reinterpret_cast<const uint2*>(recK + (int64_t)(rk0 + baseK + i) * kRecBytes + 8 * kg);
      const uint32_t xs[3][2] = {{x.x, x.y}, {x.x >> 6, x.y >> 6}, {x.x >> 12, x.y >> 12}};
      bf16x8 af[4];
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const Plane p0 = plane_of(2 * st), p1 = plane_of(2 * st + 1);
        const int i0 = p0.sh / 6, i1 = p1.sh / 6;
        af[st] = u4_to_frag(and_or(xs[i0][0], MK[p0.m], vbias), and_or(xs[i0][1], MK[p0.m], vbias),
                            and_or(xs[i1][0], MK[p1.m], vbias), and_or(xs[i1][1], MK[p1.m], vbias));
      }
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) {
        const float2 qc = qcs[cb * 64 + lane];  // (sum of q, initial accumulator)
        f32x4 cacc = {qc.y, qc.y, qc.y, qc.y};
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          cacc = M::mma(af[st], bits_to_frag(qbs[(cb * 4 + st) * QH][lane]), cacc);
          if constexpr (QSPLIT) cacc = M::mma(af[st], bits_to_frag(qbs[(cb * 4 + st) * QH + 1][lane]), cacc);
        }
        const int kap = 16 * cb + col, g = kap >> 2, grp = kap & 3;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int ii = b0 + 4 * kg + r;
          uint32_t sz = 0;
          if constexpr (LDS) sz = *reinterpret_cast<const uint32_t*>(kstb + (baseK + ii) * kRecBytes + 32 + 4 * grp);
          else if (ii < nK) sz = *reinterpret_cast<const uint32_t*>(recK + (int64_t)(rk0 + baseK + ii) * kRecBytes + 32 + 4 * grp);
          const float sc = h2f((uint16_t)(sz & 0xFFFFu)), z = h2f((uint16_t)(sz >> 16));
          const float val = quad_sum(fmaf(sc, cacc[r], z * qc.x));
          if (ii < nK && grp == 0 && g < G) wbuf[ii * BR + g] = val * a.c;
        }
      }
    };
    {
      const int nfast = max(0, min(nK, kRecCap - baseK));  // records of this wave that are staged
      int b0 = 0;
      for (; b0 + 16 <= nfast; b0 += 16) kbatch(b0, std::true_type{});
      if (b0 < nK) {
        if (baseK + nK <= kRecCap) kbatch(b0, std::true_type{});
        else for (; b0 < nK; b0 += 16) kbatch(b0, std::false_type{});
      }
    }
    __builtin_amdgcn_wave_barrier();  // this wave's buf rows written before they are read (LDS is in order per wave)

    // ---- C: logits of the lane's two tokens; tile max per q-head
    float s0[G], s1[G];
    {
      float S0[GP], S1[GP], R0[GP], R1[GP];
      ldsv<GP>(S + aK0 * GP, S0);
      ldsv<GP>(S + aK1 * GP, S1);
      ldsv<GP>(fK0 ? wbuf + rK0 * BR : zrow, R0);
      ldsv<GP>(fK1 ? wbuf + rK1 * BR : zrow, R1);
      bool hot = false;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        s0[g] = v0 ? fmaf(gK0, S0[g], R0[g]) : -INFINITY;
        s1[g] = v1 ? fmaf(gK1, S1[g], R1[g]) : -INFINITY;
        hot |= fmaxf(s0[g], s1[g]) > m_run[g] + kLazy;
      }
      // Only a logit above m_run + kLazy changes anything (the rescale below);
      // a wave holding one publishes its exact maximum, the others nothing
      // (their maxima are smaller than any such logit).
      if (__any(hot)) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const int mk = wave_max_i32(fkey(fmaxf(s0[g], s1[g])));
          if (lane == 0) atomicMax(&tmaxb[par][g], mk);
        }
      }
    }
    lds_barrier();
    // ---- D: lazy rescale (every thread takes the same decision).  The
    // probabilities are first computed with the current m_run while the
    // tile maxima are read, and again in the rare case that m_run moves.
    float pk0[BR], pk1[BR];
#pragma unroll
    for (int g = 0; g < BR; ++g) { pk0[g] = 0.0f; pk1[g] = 0.0f; }
    int tk[G];
#pragma unroll
    for (int g = 0; g < G; ++g) tk[g] = tmaxb[par][g];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      pk0[g] = exp2_fast(s0[g] - m_run[g]);
      pk1[g] = exp2_fast(s1[g] - m_run[g]);
    }
    bool any = false;
    float fct[G];
    {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float tm = fkey_inv(tk[g]);
        fct[g] = 1.0f;
        if (tm > m_run[g] + kLazy) {
          fct[g] = (m_run[g] == -INFINITY) ? 0.0f : exp2_fast(m_run[g] - tm);
          m_run[g] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, tm)));  // uniform
          any = true;
        }
      }
    }
    if (any) {
#pragma unroll
      for (int g = 0; g < G; ++g) lacc[g] *= fct[g];
#pragma unroll
      for (int g = 0; g < G; ++g)
        if (fct[g] != 1.0f)
          for (int i = threadIdx.x; i < A; i += blockDim.x)
            wi[g * A + i] = (unsigned long long)__double2ll_rn((double)(long long)wi[g * A + i] * (double)fct[g]);
#pragma unroll
      for (int rb = 0; rb < NB; ++rb) {
        const int g = 4 * rb + kg;  // accumulator rows 16rb + 4kg + r -> q-head 4rb + kg
        float f = 1.0f;
#pragma unroll
        for (int gg = 0; gg < G; ++gg) f = (gg == g) ? fct[gg] : f;
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) vacc[rb][cc] *= f;
        const int gz = (16 * rb + col) >> 2;  // z row (rb, col)
        float fz = 1.0f;
#pragma unroll
        for (int gg = 0; gg < G; ++gg) fz = (gg == gz) ? fct[gg] : fz;
        zt[rb] *= fz;
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        pk0[g] = exp2_fast(s0[g] - m_run[g]);
        pk1[g] = exp2_fast(s1[g] - m_run[g]);
      }
      lds_barrier();
    }
    // ---- E: probabilities, scatter p*gamma into w, keep p of value-flagged
    // tokens in this wave's buf rows [0, nV) and zeros in the rows after them
    // up to the next multiple of 32 (the value batches read whole batches).
    // A token past the range has p = 0 and adds 0 to w[0].
    // p <= 2 (lazy rescale), so gamma in [0, 8) keeps y = p*gamma*2^38 in
    // [0, 2^42): one f64 fma adds 1.5*2^52, which rounds y to the nearest
    // integer and leaves it in the low 51 bits (p and gamma are exact in f64,
    // so this is the only rounding).
    {
      const float gs0 = gV0 * kFxScale, gs1 = gV1 * kFxScale;
      const bool fast = __all((!v0 || (gV0 >= 0.0f && gV0 < 8.0f)) && (!v1 || (gV1 >= 0.0f && gV1 < 8.0f)));
#pragma unroll
      for (int g = 0; g < G; ++g) lacc[g] += pk0[g] + pk1[g];
      if (fast) {
        const double gd0 = (double)gV0 * kFxScaleD, gd1 = (double)gV1 * kFxScaleD;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          atomicAdd(wi + g * A + aV0,
                    (unsigned long long)__double_as_longlong(fma((double)pk0[g], gd0, kRoundMagic)) & kMagicMask);
          atomicAdd(wi + g * A + aV1,
                    (unsigned long long)__double_as_longlong(fma((double)pk1[g], gd1, kRoundMagic)) & kMagicMask);
        }
      } else {
#pragma unroll
        for (int g = 0; g < G; ++g) {
          atomicAdd(wi + g * A + aV0, fx_general(pk0[g] * gs0));
          atomicAdd(wi + g * A + aV1, fx_general(pk1[g] * gs1));
        }
      }
      if (fV0) stsv<BR>(wbuf + rV0 * BR, pk0);
      if (fV1) stsv<BR>(wbuf + rV1 * BR, pk1);
      const int zr = nV + lane;
      if (zr < ((nV + 31) & ~31)) {
        float z0[BR];
#pragma unroll
        for (int g = 0; g < BR; ++g) z0[g] = 0.0f;
        stsv<BR>(wbuf + zr * BR, z0);
      }
    }
    __builtin_amdgcn_wave_barrier();

    // ---- F: value residuals of this wave's records, 32 per MFMA K-step
    // (staged records from LDS; overflow records from the cache in a separate loop)
    auto vbatch = [&](int b0, auto from_lds) {
      constexpr bool LDS = decltype(from_lds)::value;
      uint32_t pr[4];  // code words of coordinate column `col`, record pairs
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const int r0 = b0 + 8 * kg + 2 * e2;
        uint32_t w0 = 0, w1 = 0;
        if constexpr (LDS) {
          w0 = *reinterpret_cast<const uint16_t*>(vstb + (baseV + r0) * kRecBytes + 2 * col);
          w1 = *reinterpret_cast<const uint16_t*>(vstb + (baseV + r0 + 1) * kRecBytes + 2 * col);
        } else {
          if (r0 < nV) w0 = *reinterpret_cast<const uint16_t*>(recV + (int64_t)(rv0 + baseV + r0) * kRecBytes + 2 * col);
          if (r0 + 1 < nV) w1 = *reinterpret_cast<const uint16_t*>(recV + (int64_t)(rv0 + baseV + r0 + 1) * kRecBytes + 2 * col);
        }
        pr[e2] = w0 | (w1 << 16);
      }
      // A operands: row (4g + grp) = 16rb + col, records b0 + 8kg + e; the
      // buf rows give p = 0 to padded q-heads and to records past nV (the
      // staged records there are finite: other waves' or zeros)
      bf16x8 ahi[NB], alo[NB];
      f32x4 zb[NB];  // -128 * row sums of A: cancels the code bias
#pragma unroll
      for (int rb = 0; rb < NB; ++rb) {
        const int g = (16 * rb + col) >> 2, grp = col & 3;
        float ps[8];
        float zsum = zt[rb];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int rr = b0 + 8 * kg + e;
          const float pv = wbuf[rr * BR + g];
          uint32_t sz = 0;
          if constexpr (LDS) sz = *reinterpret_cast<const uint32_t*>(vstb + (baseV + rr) * kRecBytes + 32 + 4 * grp);
          else if (rr < nV) sz = *reinterpret_cast<const uint32_t*>(recV + (int64_t)(rv0 + baseV + rr) * kRecBytes + 32 + 4 * grp);
          ps[e] = fmaf(pv, h2f((uint16_t)(sz & 0xFFFFu)), 0.0f);
          zsum = fmaf(pv, h2f((uint16_t)(sz >> 16)), zsum);
        }
        zt[rb] = zsum;
        uint32_t hp[4], lp[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t hb = bf16_pack(ps[2 * k], ps[2 * k + 1]);
          const float d0 = ps[2 * k] - __uint_as_float(hb << 16);
          const float d1 = ps[2 * k + 1] - __uint_as_float(hb & 0xFFFF0000u);
          hp[k] = hb;
          lp[k] = bf16_pack(d0, d1);
        }
        ahi[rb] = u4_to_frag(hp[0], hp[1], hp[2], hp[3]);
        alo[rb] = u4_to_frag(lp[0], lp[1], lp[2], lp[3]);
        zb[rb] = M::mma(ahi[rb], bm128, f32x4{0, 0, 0, 0});
        zb[rb] = M::mma(alo[rb], bm128, zb[rb]);
      }
      const uint32_t ps6[4] = {pr[0] >> 6, pr[1] >> 6, pr[2] >> 6, pr[3] >> 6};
      const uint32_t ps12[4] = {pr[0] >> 12, pr[1] >> 12, pr[2] >> 12, pr[3] >> 12};
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) {
        const Plane pl = plane_of(cc);
        const uint32_t* src = pl.sh == 0 ? pr : pl.sh == 6 ? ps6 : ps12;
        const bf16x8 bfr = u4_to_frag(and_or(src[0], MK[pl.m], vbias), and_or(src[1], MK[pl.m], vbias),
                                      and_or(src[2], MK[pl.m], vbias), and_or(src[3], MK[pl.m], vbias));
#pragma unroll
        for (int rb = 0; rb < NB; ++rb) {
          f32x4 t = M::mma(ahi[rb], bfr, zb[rb]);
          t = M::mma(alo[rb], bfr, t);
          vacc[rb][cc] += t[cc >> 1];
        }
      }
    };
    {
      const int nfast = max(0, min(nV, kRecCap - baseV));
      int b0 = 0;
      for (; b0 + 32 <= nfast; b0 += 32) vbatch(b0, std::true_type{});
      if (b0 < nV) {
        if (baseV + nV <= kRecCap) vbatch(b0, std::true_type{});
        else for (; b0 < nV; b0 += 32) vbatch(b0, std::false_type{});
      }
    }
    lds_barrier();  // staged records and buf are reused by the next tile
  }
  }

  // ---- epilogue: reduce over lanes and waves, write this range's partial state
  __shared__ float lsum[kWaves][G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float l = wave_sum(lacc[g]);
    if (lane == 0) lsum[wave][g] = l;
  }
  float* accs = buf;  // [G][D]
  for (int i = threadIdx.x; i < G * D; i += blockDim.x) accs[i] = 0.0f;
  __syncthreads();
#pragma unroll
  for (int rb = 0; rb < NB; ++rb) {
    float z = zt[rb];
    z += __shfl_xor(z, 16, 64);
    z += __shfl_xor(z, 32, 64);
    const int g = (16 * rb + col) >> 2;
    if (kg == 0 && g < G) atomicAdd(&zt_s[g * 4 + (col & 3)], z);
    // lane (col j, kg) of column block cc holds rows 16rb + 4kg + r = (q-head 4rb + kg, group r);
    // only group r == cc/2 covers coordinate j + 16cc.
    const int gq = 4 * rb + kg;
    if (gq < G)
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) {
        atomicAdd(&accs[gq * D + col + 16 * cc], vacc[rb][cc] * kPlaneInv[plane_of(cc).m]);
      }
  }
  // ---- w V on MFMA: wave w takes coordinates 16w .. 16w+15 (rows = q-heads,
  // K = anchors, columns = coordinates); w in bf16 hi + lo for bf16 data
  static_assert(kWaves * 16 == D, "one 16-coordinate block per wave");
  const int d = 16 * wave + col;
  f32x4 ov = {0, 0, 0, 0};
  {
    using MV = Mfma<DT>;
    const T* AV = reinterpret_cast<const T*>(base + a.off_av) + (int64_t)h * A * D;
#pragma unroll 4
    for (int a0 = 0; a0 < A; a0 += MV::KSTEP) {
      const int ab = a0 + kg * MV::KW;
      if constexpr (DT == ANCHORKV_BF16) {
        float wv[8];
        uint32_t vb[4];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          wv[e] = (col < G && ab + e < A) ? (float)((double)(long long)wi[col * A + ab + e] * kFxInv) : 0.0f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t v0 = ab + 2 * k < A ? (uint32_t)AV[(int64_t)(ab + 2 * k) * D + d] : 0u;
          const uint32_t v1 = ab + 2 * k + 1 < A ? (uint32_t)AV[(int64_t)(ab + 2 * k + 1) * D + d] : 0u;
          vb[k] = v0 | (v1 << 16);
        }
        uint32_t hp[4], lp[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          hp[k] = bf16_pack(wv[2 * k], wv[2 * k + 1]);
          lp[k] = bf16_pack(wv[2 * k] - __uint_as_float(hp[k] << 16), wv[2 * k + 1] - __uint_as_float(hp[k] & 0xFFFF0000u));
        }
        const bf16x8 bv = u4_to_frag(vb[0], vb[1], vb[2], vb[3]);
        ov = MV::mma(u4_to_frag(hp[0], hp[1], hp[2], hp[3]), bv, ov);
        ov = MV::mma(u4_to_frag(lp[0], lp[1], lp[2], lp[3]), bv, ov);
      } else {
        const float wv = (col < G && ab < A) ? (float)((double)(long long)wi[col * A + ab] * kFxInv) : 0.0f;
        const float vv = ab < A ? Elem<DT>::f(AV[(int64_t)ab * D + d]) : 0.0f;
        ov = MV::mma(wv, vv, ov);
      }
    }
  }
  // (max, sum) of this range per q-head
  __shared__ float ml_s[2][kMaxG];
  if (threadIdx.x < G) {
    const int g = threadIdx.x;
    float l = 0.0f;
    for (int w2 = 0; w2 < kWaves; ++w2) l += lsum[w2][g];
    float m = -INFINITY;
#pragma unroll
    for (int gg = 0; gg < G; ++gg) m = (gg == g) ? m_run[gg] : m;
    ml_s[0][g] = m;
    ml_s[1][g] = l;
  }
  __syncthreads();
  // lane (col, kg) holds rows g = 4kg + r of coordinate d
  float val[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int g = 4 * kg + r;
    val[r] = g < G ? ov[r] + accs[g * D + d] + zt_s[g * 4 + d / 32] : 0.0f;
  }
  if (a.S2 == 1 && !a.force_part) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int g = 4 * kg + r;
      if (g < G) a.o[(uh * G + g) * D + d] = val[r] / ml_s[1][g];
    }
    return;
  }
  // several ranges per head, or a tail to follow: publish this one (merged by k_dec_merge)
  const int64_t ps = uh * a.S2 + sp;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int g = 4 * kg + r;
    if (g < G) a.part_acc[(ps * G + g) * D + d] = val[r];
  }
  if (threadIdx.x < G) a.part_ml[ps * G + threadIdx.x] = make_float2(ml_s[0][threadIdx.x], ml_s[1][threadIdx.x]);
}

// Per (unit, head) with several token ranges (and an optional tail partial):
// o = sum_s f_s acc_s / sum_s f_s l_s with f_s = 2^(m_s - max m).  One thread
// per (q-head, coordinate).
__global__ __launch_bounds__(256) void k_dec_merge(const float2* part_ml, const float* part_acc, const float2* tail_ml,
                                                  const float* tail_acc, float* o, int G, int S2, int St) {
  const int64_t uh = blockIdx.x;
  for (int i = threadIdx.x; i < G * kHeadDim; i += blockDim.x) {
    const int g = i / kHeadDim, d = i % kHeadDim;
    float M = -INFINITY;
    for (int s = 0; s < S2; ++s) M = fmaxf(M, part_ml[(uh * S2 + s) * G + g].x);
    for (int s = 0; s < St; ++s) M = fmaxf(M, tail_ml[(uh * St + s) * G + g].x);
    float L = 0.0f, acc = 0.0f;
    for (int s = 0; s < S2; ++s) {
      const float2 v = part_ml[(uh * S2 + s) * G + g];
      const float f = v.x == -INFINITY ? 0.0f : exp2_fast(v.x - M);
      L += f * v.y;
      acc = fmaf(f, part_acc[((uh * S2 + s) * G + g) * kHeadDim + d], acc);
    }
    for (int s = 0; s < St; ++s) {
      const float2 v = tail_ml[(uh * St + s) * G + g];
      const float f = v.x == -INFINITY ? 0.0f : exp2_fast(v.x - M);
      L += f * v.y;
      acc = fmaf(f, tail_acc[((uh * St + s) * G + g) * kHeadDim + d], acc);
    }
    o[(uh * G + g) * kHeadDim + d] = acc / L;
  }
}

// One tail tile's loads: VPT value chunks of the thread, the lane's key-row quarter.
template <typename T, int VPT, int KPL, int CPR, int EPC>
__device__ __forceinline__ void tail_load(uint4 (&vr)[VPT], uint4 (&kr)[KPL], const T* Vp, const T* Kp, int t0,
                                          int last, int tid, int jt, int qoff) {
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int i = tid + 256 * k;
    vr[k] = *reinterpret_cast<const uint4*>(Vp + (int64_t)min(t0 + i / CPR, last) * kHeadDim + (i % CPR) * EPC);
  }
  const T* row = Kp + (int64_t)min(t0 + jt, last) * kHeadDim + qoff;
#pragma unroll
  for (int k = 0; k < KPL; ++k) kr[k] = *reinterpret_cast<const uint4*>(row + k * EPC);
}

// Exact tail of one (unit, KV head): tokens appended after the one-shot
// compression and kept at the cache's element type (AnchorKV-adapted page,
// "Adaptation notes").  Workgroup s of the head takes tail range s (whole
// 64-token tiles).  Per tile: all key and value loads are issued at once (16
// bytes per lane; rows past the range clamped to its last row, so no
// branches; other resident workgroups cover the latency); the value rows go
// to LDS; lane (token j, quarter) of wave w dots a quarter of key row 16w + j
// with every q-head (quad sums); wave w raises the running maxima of q-heads
// w and w + 4 and turns their logits (c <q, k>, log2 domain) into
// probabilities; thread (half, d)
// adds p v for coordinate d of q-heads half, half + 2, ...  Writes the range's
// (max, sum, unnormalised output) partial for k_dec_merge.
template <int DT>
__global__ __launch_bounds__(256) void k_dec_tail(const void* q, const void* Kt, const void* Vt, int n_tail,
                                                 int tail_cap, int G, int St, float c, float2* tml, float* tacc) {
  using T = typename Elem<DT>::T;
  constexpr int D = kHeadDim, TT = 64, EPC = 16 / (int)sizeof(T), CPR = D / EPC;
  constexpr int VPT = TT * CPR / 256;   // 16-byte value chunks per thread and tile
  constexpr int KPL = 32 / EPC;         // 16-byte chunks of a key-row quarter
  __shared__ float qs[kMaxG][D];
  __shared__ __align__(16) T vs[TT][D];
  __shared__ float ps[kMaxG][TT];
  __shared__ float fr[kMaxG], mrun[kMaxG], lrun[kMaxG];
  const int s = blockIdx.x % St;
  const int64_t uh = blockIdx.x / St;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int span = ((n_tail + St - 1) / St + TT - 1) / TT * TT;
  const int t_beg = min(n_tail, s * span), t_end = min(n_tail, t_beg + span);
  const T* qp = reinterpret_cast<const T*>(q) + uh * G * D;
  for (int i = tid; i < G * D; i += 256) qs[i / D][i % D] = Elem<DT>::f(qp[i]);
  if (tid < kMaxG) { mrun[tid] = -INFINITY; lrun[tid] = 0.0f; }
  const T* Kp = reinterpret_cast<const T*>(Kt) + uh * (int64_t)tail_cap * D;
  const T* Vp = reinterpret_cast<const T*>(Vt) + uh * (int64_t)tail_cap * D;
  const int d = tid & (D - 1), half = tid >> 7;
  const int jt = 16 * wave + (lane >> 2), qq = lane & 3;   // logit lanes: token, quarter of the row
  float acc[kMaxG / 2];
#pragma unroll
  for (int k = 0; k < kMaxG / 2; ++k) acc[k] = 0.0f;
  const int qoff = 32 * qq;
  __syncthreads();
  for (int t0 = t_beg; t0 < t_end; t0 += TT) {
    const int nt = min(TT, t_end - t0);
    // all of the tile's key and value loads at once (rows clamped: no branches)
    uint4 vr[VPT], kr4[KPL];
    tail_load<T, VPT, KPL, CPR, EPC>(vr, kr4, Vp, Kp, t0, t_end - 1, tid, jt, qoff);
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const int i = tid + 256 * k, r = i / CPR, ch = i % CPR;
      *reinterpret_cast<uint4*>(&vs[r][ch * EPC]) = vr[k];
    }
    float sg[kMaxG];
#pragma unroll
    for (int g = 0; g < kMaxG; ++g) sg[g] = 0.0f;
#pragma unroll
    for (int k = 0; k < KPL; ++k) {
      const uint4 raw = kr4[k];
      T kv[EPC];
      __builtin_memcpy(kv, &raw, 16);
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        const float kf = Elem<DT>::f(kv[e]);
#pragma unroll
        for (int g = 0; g < kMaxG; ++g)
          if (g < G) sg[g] = fmaf(qs[g][32 * qq + k * EPC + e], kf, sg[g]);
      }
    }
#pragma unroll
    for (int g = 0; g < kMaxG; ++g)
      if (g < G) {
        const float v = quad_sum(sg[g]);
        if (qq == 0) ps[g][jt] = jt < nt ? v * c : -INFINITY;
      }
    __syncthreads();
    for (int g = wave; g < G; g += 4) {   // wave w: q-heads w, w + 4
      const float x = ps[g][lane];
      const float mn = fmaxf(mrun[g], wave_max(x));
      const float f = mrun[g] == -INFINITY ? 0.0f : exp2_fast(mrun[g] - mn);
      const float p = lane < nt ? exp2_fast(x - mn) : 0.0f;
      ps[g][lane] = p;
      const float sum = wave_sum(p);
      if (lane == 0) { fr[g] = f; lrun[g] = fmaf(lrun[g], f, sum); mrun[g] = mn; }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kMaxG / 2; ++k) {
      const int g = half + 2 * k;
      if (g < G) {
        // all TT rows: past nt, p = 0 and the value rows are clamped copies
        float a = acc[k] * fr[g];
#pragma unroll 16
        for (int t = 0; t < TT; ++t) a = fmaf(ps[g][t], Elem<DT>::f(vs[t][d]), a);
        acc[k] = a;
      }
    }
    __syncthreads();   // vs, ps, fr are rewritten by the next tile
  }
  const int64_t slot = uh * St + s;
  if (tid < G) tml[slot * G + tid] = make_float2(mrun[tid], lrun[tid]);
#pragma unroll
  for (int k = 0; k < kMaxG / 2; ++k)
    if (half + 2 * k < G) tacc[(slot * G + half + 2 * k) * D + d] = acc[k];
}

// The bf16 tail on MFMA, same ranges, tiles and partials as k_dec_tail:
// logits with rows = the wave's 16 tokens (key rows as A fragments straight
// from memory), columns = q-heads (the query as B fragments, exact bf16);
// p v with rows = q-heads (p as bf16 hi + lo from LDS), K = 32 tokens,
// columns = 16 coordinates (value B fragments gathered from the LDS tile);
// wave w owns coordinate blocks 2w and 2w + 1.
__global__ __launch_bounds__(256) void k_dec_tail_bf16(const void* q, const void* Kt, const void* Vt, int n_tail,
                                                      int tail_cap, int G, int St, float c, float2* tml,
                                                      float* tacc) {
  using M = Mfma<ANCHORKV_BF16>;
  constexpr int D = kHeadDim, TT = 64, CPR = D / 8, VPT = TT * CPR / 256;
  __shared__ __align__(16) uint16_t vs[TT][D];
  __shared__ __align__(16) float ps[16][TT];   // rows >= G stay zero
  __shared__ float fr[kMaxG], mrun[kMaxG], lrun[kMaxG];
  const int s = blockIdx.x % St;
  const int64_t uh = blockIdx.x / St;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, kg = lane >> 4;
  const int span = ((n_tail + St - 1) / St + TT - 1) / TT * TT;
  const int t_beg = min(n_tail, s * span), t_end = min(n_tail, t_beg + span);
  const uint16_t* qp = reinterpret_cast<const uint16_t*>(q) + uh * G * D;
  const uint16_t* Kp = reinterpret_cast<const uint16_t*>(Kt) + uh * (int64_t)tail_cap * D;
  const uint16_t* Vp = reinterpret_cast<const uint16_t*>(Vt) + uh * (int64_t)tail_cap * D;
  bf16x8 qf[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) qf[st] = col < G ? M::load(qp + col * D + st * 32 + kg * 8) : M::zero();
  for (int i = tid; i < 16 * TT; i += 256) ps[i / TT][i % TT] = 0.0f;
  if (tid < kMaxG) { mrun[tid] = -INFINITY; lrun[tid] = 0.0f; }
  f32x4 oacc[2] = {f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}};
  __syncthreads();
  for (int t0 = t_beg; t0 < t_end; t0 += TT) {
    const int nt = min(TT, t_end - t0), last = t_end - 1;
    // all of the tile's loads at once (rows clamped to the range: no branches)
    uint4 vr[VPT];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const int i = tid + 256 * k;
      vr[k] = *reinterpret_cast<const uint4*>(Vp + (int64_t)min(t0 + i / CPR, last) * D + (i % CPR) * 8);
    }
    const uint16_t* kr = Kp + (int64_t)min(t0 + 16 * wave + col, last) * D + kg * 8;
    bf16x8 kf[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) kf[st] = M::load(kr + st * 32);
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const int i = tid + 256 * k;
      *reinterpret_cast<uint4*>(&vs[i / CPR][(i % CPR) * 8]) = vr[k];
    }
    f32x4 acc = {0, 0, 0, 0};
#pragma unroll
    for (int st = 0; st < 4; ++st) acc = M::mma(kf[st], qf[st], acc);
    if (col < G)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * wave + 4 * kg + r;
        ps[col][j] = j < nt ? acc[r] * c : -INFINITY;
      }
    __syncthreads();
    for (int g = wave; g < G; g += 4) {   // wave w: q-heads w, w + 4
      const float x = ps[g][lane];
      const float mn = fmaxf(mrun[g], wave_max(x));
      const float f = mrun[g] == -INFINITY ? 0.0f : exp2_fast(mrun[g] - mn);
      const float p = lane < nt ? exp2_fast(x - mn) : 0.0f;
      ps[g][lane] = p;
      const float sum = wave_sum(p);
      if (lane == 0) { fr[g] = f; lrun[g] = fmaf(lrun[g], f, sum); mrun[g] = mn; }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int g = 4 * kg + r;
      const float f = g < G ? fr[g] : 0.0f;
      oacc[0][r] *= f;
      oacc[1][r] *= f;
    }
#pragma unroll
    for (int ks = 0; ks < TT / 32; ++ks) {
      float p8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) p8[e] = ps[col][ks * 32 + kg * 8 + e];
      bf16x8 ph, pl;
      split8(p8, ph, pl);
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int d = (2 * wave + b) * 16 + col;
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          w[e] = (uint32_t)vs[ks * 32 + kg * 8 + 2 * e][d] | ((uint32_t)vs[ks * 32 + kg * 8 + 2 * e + 1][d] << 16);
        const bf16x8 vb = bits_to_frag(make_uint4(w[0], w[1], w[2], w[3]));
        oacc[b] = M::mma(ph, vb, oacc[b]);
        oacc[b] = M::mma(pl, vb, oacc[b]);
      }
    }
    __syncthreads();   // vs, ps, fr are rewritten by the next tile
  }
  const int64_t slot = uh * St + s;
  if (tid < G) tml[slot * G + tid] = make_float2(mrun[tid], lrun[tid]);
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int g = 4 * kg + r;
      if (g < G) tacc[(slot * G + g) * D + (2 * wave + b) * 16 + col] = oacc[b][r];
    }
}

// Raise a kernel's dynamic-LDS limit to `bytes` (once per larger value).

static size_t stream_lds(int G, int A, int KP, bool qsplit) {
  const size_t GP = G <= 1 ? 1 : G <= 2 ? 2 : G <= 4 ? 4 : 8;
  const size_t NB = (4 * (size_t)G + 15) / 16;
  return sizeof(float) * ((3 * GP * A + 3) & ~(size_t)3) + sizeof(float) * (size_t)std::max<size_t>(kTile * 4 * NB, 2048) +
         2 * 512 * (size_t)KP * sizeof(uint4) + (size_t)kRecPad * kRecBytes + NB * 4 * (qsplit ? 2 : 1) * 64 * sizeof(uint4) +
         NB * 64 * sizeof(float2);
}
constexpr size_t kLdsLimit = 158 * 1024;  // dynamic part; the static part is under 2 KB of the 160 KB

template <int DT, int G, int KP, int DEPTH, int WPE>
static int launch_stream_kp(const DecArgs& a, unsigned grid, hipStream_t st) {
  static size_t done = 0;
  const size_t lds = stream_lds(G, a.A, KP, DT == ANCHORKV_F32);
  if (lds > kLdsLimit) return fail(ANCHORKV_E_SHAPE, "decode: q_per_kv * anchors too large for LDS");
  if (int rc = set_dyn_lds(reinterpret_cast<const void*>(&k_dec_stream<DT, G, KP, DEPTH, WPE>), lds, &done)) return rc;
  k_dec_stream<DT, G, KP, DEPTH, WPE><<<grid, 64 * kWaves, lds, st>>>(a);
  AKV_CHECK_LAUNCH("k_dec_stream");
  return 0;
}

// Staged 16-byte chunks per thread and side (KP; 512*KP*16/48 records per
// tile) from the average number of residual records per 1024-token tile:
// larger staging costs registers and LDS, records beyond it are read from
// the cache directly.
// Falls back to the largest staging that fits LDS (KP = 1 always fits a plan
// that anchorkv_plan accepted).
static int decode_kp(int G, int A, bool f32, int64_t R_K, int64_t R_V, int64_t H, int64_t C) {
  if (G > 4) return 1;
  const int64_t per = std::max(R_K, R_V) / std::max<int64_t>(1, H * C);
  int kp = per <= 150 ? 1 : per <= 300 ? 2 : 3;
  while (kp > 1 && stream_lds(G, A, kp, f32) > kLdsLimit) --kp;
  return kp;
}

// Up to 4 q-heads per KV head: four waves per SIMD (two workgroups per CU);
// more q-heads: two waves per SIMD (one workgroup per CU, LDS-bound).
template <int DT, int G>
static int launch_stream(const DecArgs& a, unsigned grid, hipStream_t st) {
  if constexpr (G <= 4) {
    switch (decode_kp(G, a.A, DT == ANCHORKV_F32, a.R_K, a.R_V, a.H, a.C)) {
      case 1: return launch_stream_kp<DT, G, 1, 1, 4>(a, grid, st);
      case 2: return launch_stream_kp<DT, G, 2, 1, 4>(a, grid, st);
      default: return launch_stream_kp<DT, G, 3, 1, 4>(a, grid, st);
    }
  } else {
    return launch_stream_kp<DT, G, 1, 2, 2>(a, grid, st);
  }
}

template <int DT>
static int decode_impl(const anchorkv_plan_info& p, const void* cache_v, const void* q, float* o, void* ws_v,
                       hipStream_t st, const void* K_tail = nullptr, const void* V_tail = nullptr, int n_tail = 0,
                       int tail_cap = 0) {
  const uint8_t* cache = reinterpret_cast<const uint8_t*>(cache_v);
  uint8_t* ws = reinterpret_cast<uint8_t*>(ws_v);
  const DecodeWs w = decode_ws_layout(p);
  const int U = p.units, H = p.H, G = p.G, A = p.A, S2 = w.S2;
  if (G > kMaxG) return fail(ANCHORKV_E_SHAPE, "decode supports q_per_kv <= %d", kMaxG);
  if (S2 > 64) return fail(ANCHORKV_E_SHAPE, "decode: too many splits");
  if (stream_lds(G, A, 1, DT == ANCHORKV_F32) > kLdsLimit) return fail(ANCHORKV_E_SHAPE, "decode: q_per_kv * anchors too large for LDS");
  if (p.n_chunks > 128 * S2) return fail(ANCHORKV_E_SHAPE, "decode: too many chunks per range");
  prof_call_begin(st);
  DecArgs a;
  a.q = q; a.cache = cache; a.stride = p.unit_stride; a.off_words = p.off_words; a.off_rk = p.off_res_k;
  a.off_rv = p.off_res_v; a.off_ck = p.off_chunk_k; a.off_cv = p.off_chunk_v;
  a.off_ak = p.off_anchor_k; a.off_av = p.off_anchor_v;
  a.part_ml = reinterpret_cast<float2*>(ws + w.part_ml);
  a.part_acc = reinterpret_cast<float*>(ws + w.part_acc);
  a.o = o;
  a.H = H; a.N = p.N; a.A = A; a.C = p.n_chunks; a.S2 = S2; a.cps = (p.n_chunks + S2 - 1) / S2;
  a.c = kLog2e / sqrtf((float)kHeadDim);
  a.R_K = p.R_K; a.R_V = p.R_V;
  a.force_part = n_tail > 0 ? 1 : 0;
  const unsigned grid = (unsigned)((int64_t)U * H * S2);
  int rc = 0;
  switch (G) {
    case 1: rc = launch_stream<DT, 1>(a, grid, st); break;
    case 2: rc = launch_stream<DT, 2>(a, grid, st); break;
    case 3: rc = launch_stream<DT, 3>(a, grid, st); break;
    case 4: rc = launch_stream<DT, 4>(a, grid, st); break;
    case 5: rc = launch_stream<DT, 5>(a, grid, st); break;
    case 6: rc = launch_stream<DT, 6>(a, grid, st); break;
    case 7: rc = launch_stream<DT, 7>(a, grid, st); break;
    default: rc = launch_stream<DT, 8>(a, grid, st); break;
  }
  if (rc) return rc;
  if (n_tail > 0) {
    prof_mark(st, "dec_stream");
    float2* tml = reinterpret_cast<float2*>(ws + w.tail_ml);
    float* tacc = reinterpret_cast<float*>(ws + w.tail_acc);
    if constexpr (DT == ANCHORKV_BF16)
      k_dec_tail_bf16<<<(unsigned)((int64_t)U * H * w.St), 256, 0, st>>>(q, K_tail, V_tail, n_tail, tail_cap, G,
                                                                         w.St, a.c, tml, tacc);
    else
      k_dec_tail<DT><<<(unsigned)((int64_t)U * H * w.St), 256, 0, st>>>(q, K_tail, V_tail, n_tail, tail_cap, G, w.St,
                                                                          a.c, tml, tacc);
    AKV_CHECK_LAUNCH("k_dec_tail");
    k_dec_merge<<<(unsigned)((int64_t)U * H), 256, 0, st>>>(a.part_ml, a.part_acc, tml, tacc, o, G, S2, w.St);
    AKV_CHECK_LAUNCH("k_dec_merge");
    prof_mark(st, "dec_tail");
    return 0;
  }
  if (S2 > 1) {
    k_dec_merge<<<(unsigned)((int64_t)U * H), 256, 0, st>>>(a.part_ml, a.part_acc, nullptr, nullptr, o, G, S2, 0);
    AKV_CHECK_LAUNCH("k_dec_merge");
  }
  prof_mark(st, "dec_stream");
  return 0;
}

int decode_blocks_per_cu(int G, int A, bool f32, int64_t R_K, int64_t R_V, int64_t H, int64_t C) {
  // G <= 4 runs at four waves per SIMD (two 8-wave workgroups) when two
  // copies of its LDS fit the 160 KB (static part under 2 KB each)
  const int kp = decode_kp(G, A, f32, R_K, R_V, H, C);
  return (G <= 4 && 2 * (stream_lds(G, A, kp, f32) + 2048) <= 160 * 1024) ? 2 : 1;
}

int decode_supports(const anchorkv_plan_info& p) {
  if (p.G > kMaxG) return fail(ANCHORKV_E_SHAPE, "anchorkv_plan: decode supports q_per_kv <= %d", kMaxG);
  if (stream_lds(p.G, p.A, 1, p.dtype == ANCHORKV_F32) > kLdsLimit)
    return fail(ANCHORKV_E_SHAPE, "anchorkv_plan: %d anchors x %d q-heads exceed the decode kernel's LDS", p.A, p.G);
  if (p.decode_splits > 64 || p.n_chunks > 128 * p.decode_splits)
    return fail(ANCHORKV_E_SHAPE, "anchorkv_plan: n_tokens %d too large for the decode ranges", p.N);
  return 0;
}

int run_decode(const anchorkv_plan_info& p, const void* cache, const void* q, float* o, void* ws, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (p.dtype == ANCHORKV_BF16) return decode_impl<ANCHORKV_BF16>(p, cache, q, o, ws, st);
  return decode_impl<ANCHORKV_F32>(p, cache, q, o, ws, st);
}

int run_decode_tail(const anchorkv_plan_info& p, const void* cache, const void* q, const void* K_tail,
                    const void* V_tail, int n_tail, int tail_cap, float* o, void* ws, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (p.dtype == ANCHORKV_BF16)
    return decode_impl<ANCHORKV_BF16>(p, cache, q, o, ws, st, K_tail, V_tail, n_tail, tail_cap);
  return decode_impl<ANCHORKV_F32>(p, cache, q, o, ws, st, K_tail, V_tail, n_tail, tail_cap);
}

}  // namespace akv
