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
// constant part is cancelled exactly.  Keys: rows = (q-head, group),
// columns = records, so one 16x16 tile serves 4 q-heads x 4 groups and a
// lane holds the four groups of one q-head and record.  Values:
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
#include <mutex>
#include <type_traits>

namespace akv {


constexpr int kMaxG = 8;          // q-heads per KV head supported by decode
constexpr int kTile = 1024;       // tokens per tile (= residual-offset chunk)
constexpr uint32_t kCodeBias = 0x43004300u;  // bf16 pair (128, 128)
constexpr float kFxScale = 0x1p38f;               // fixed-point scale of the w scatter
constexpr double kFxScaleD = 0x1p38;
constexpr double kFxInv = 0x1p-38;
constexpr double kRoundMagic = 0x1.8p52;           // x + 1.5*2^52 rounds x (|x| < 2^51) to an integer
constexpr unsigned long long kMagicMask = 0x0007FFFFFFFFFFFFull;  // low 51 bits: that integer, for x >= 0
constexpr float kLazy = 1.0f;                      // rescale when a logit passes m_run + kLazy (log2 units)

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
  int G;              // q-heads per KV head
  int force_part;    // publish partials even with one range (a tail follows)
  int joint, R_total; // one record section for both sides (keys first), R_total records
  int codec;          // residual codec of the cache (anchorkv_codec)
  uint4 signs;        // rotation signs of the Hadamard / Lloyd-Max codec
  float c;
  int rope;           // keys stored pre-RoPE (decoded by k_dec_rope)
  float rope_theta;   // their rotary base
};

// Hadamard / Lloyd-Max codec (Pith review of AnchorKV, "Referee Report"
// summary and "Assumptions & free parameters"): level(c) = -l2 + (l2 - l1) c
// + (3 l1 - l2) hi(c) with hi(c) the high bit of the 2-bit code, exact for
// the four levels -l2, -l1, l1, l2; the MFMAs produce sums over the codes and
// over their high bits.
constexpr float kLmL1 = 0.45278002f, kLmL2 = 1.5104176f;
constexpr float kLmAlpha = kLmL2 - kLmL1;              // weight of the code
constexpr float kLmBeta = 0.5f * (3.0f * kLmL1 - kLmL2);   // weight of the high-bit plane (which carries 2 hi)
// sign of coordinate i from the 128-bit mask
__device__ __forceinline__ float sign_of(uint4 s, int i) {
  const uint32_t w = i < 32 ? s.x : i < 64 ? s.y : i < 96 ? s.z : s.w;
  return (w >> (i & 31)) & 1u ? -1.0f : 1.0f;
}

__device__ __forceinline__ bf16x8 u4_to_frag(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return bits_to_frag(make_uint4(a, b, c, d));
}
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
__device__ __forceinline__ bf16x4 u2_to_frag4(uint32_t a, uint32_t b) { return __builtin_bit_cast(bf16x4, make_uint2(a, b)); }
// 16x16x16 bf16 MFMA (K = 16: lane (col, kg) holds K indices 4kg .. 4kg + 3)
__device__ __forceinline__ f32x4 mma16k(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
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

// LDS of the stream kernel (bytes from the start of the dynamic region), for
// NW waves of 64 * (16 / NW) tokens each per 1024-token tile.  Main phase:
// w [G][A] u64 | S [A][GP] f32 | rows [1024][BR] f32 (each wave its own
// 1024 / NW rows) | K-batch query fragments [NB*4*QH][64] uint4 | their column
// sums [NB][64] float2.  Epilogue (after the last read of w): the per-wave
// partial outputs [NW][G][D], the parts of w V [NW / 8][G][D], the zero-point
// sums [NW][4 BR] and the softmax sums [NW][GP] reuse the region.
struct DecLds {
  size_t S, rows, qbs, qcs, main;
  size_t pv, pwv, pz, pl, prot, epi;
  size_t total;
};
__host__ __device__ constexpr size_t lds_align(size_t x) { return (x + 15) & ~(size_t)15; }
__host__ __device__ inline DecLds dec_lds(int G, int A, bool qsplit, int NW, int codec = 0) {
  const size_t GP = G <= 1 ? 1 : G <= 2 ? 2 : G <= 4 ? 4 : 8;
  const bool hlm = codec == ANCHORKV_CODEC_HADAMARD_LM;
  // Hadamard / Lloyd-Max: one 16-column block (q-head, hi / lo part of the
  // rotated query) and rows of GP floats
  const size_t NB = hlm ? 1 : (4 * (size_t)G + 15) / 16, BR = hlm ? GP : 4 * NB;
  const size_t QH = (qsplit && !hlm) ? 2 : 1;
  DecLds L{};
  L.S = lds_align(8 * (size_t)G * A);
  L.rows = L.S + lds_align(4 * GP * (size_t)A);
  L.qbs = L.rows + (size_t)kTile * BR * 4;
  L.qcs = L.qbs + NB * 4 * QH * 64 * 16;
  L.main = L.qcs + NB * 64 * 8;
  L.pv = 0;
  L.pwv = L.pv + (size_t)NW * G * kHeadDim * 4;
  L.pz = L.pwv + (size_t)(NW / 8) * G * kHeadDim * 4;
  L.pl = L.pz + (size_t)NW * BR * 4 * 4;
  L.prot = L.pl + lds_align((size_t)NW * GP * 4);
  L.epi = L.prot + (hlm ? (size_t)G * kHeadDim * 4 : 0);
  L.total = L.main > L.epi ? L.main : L.epi;
  return L;
}

// One workgroup of NW waves per (unit, head, range of 1024-token chunks).
// Wave w owns tokens w*TT .. w*TT + TT - 1 of every tile (TT = 1024 / NW),
// TPL = TT / 64 adjacent tokens per lane: NW = 16 (one token per lane, 1024
// threads, one workgroup per compute unit) or NW = 8 (two tokens per lane,
// two workgroups per compute unit when their LDS fits).  Per tile there is
// one workgroup barrier, between the logits (a wave publishes its maxima
// only when a logit passes m_run + kLazy) and the softmax weights;
// everything else a wave needs is its own:
//  * the residual records of a wave's flagged tokens are a contiguous run of
//    the tile's records; the run starts at the tile's chunk offset plus the
//    flagged counts of the waves before it, which every wave publishes a tile
//    ahead (its pointer words are loaded two tiles ahead);
//  * the first 16 key records and 16 value records of the run are loaded into
//    registers a tile ahead, directly in MFMA operand layout (range-checked
//    buffer loads: records past the run read as zeros); more are read when
//    needed;
//  * key-residual logits and the weights of value-flagged tokens pass through
//    rows of LDS private to the wave;
//  * the tile maxima are triple-buffered, so resetting the one for the next
//    tile cannot race with a wave still reading the previous one.
// The epilogue sums the waves' partial outputs in a fixed order (no float
// atomics), so the output does not depend on the order the waves ran in.
template <int DT, int G, int NW, int CD>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(4))) void k_dec_stream(DecArgs a) {
  using T = typename Elem<DT>::T;
  using M = Mfma<ANCHORKV_BF16>;
  constexpr int D = kHeadDim;
  constexpr int TT = kTile / NW;                 // tokens per wave per tile
  constexpr int TPL = TT / 64;                   // tokens per lane (adjacent)
  static_assert(TPL == 1 || TPL == 2, "one or two tokens per lane");
  // Hadamard / Lloyd-Max codec: the key MFMA columns are (q-head, hi / lo
  // bf16 part of the rotated query), the value MFMA rows (q-head, hi / lo
  // part of p * sigma); one 16-wide block for up to 8 q-heads
  constexpr bool HLM = CD == ANCHORKV_CODEC_HADAMARD_LM;
  constexpr int RB = HLM ? kRecBytesHlm : kRecBytes;   // bytes per residual record
  constexpr int GP = kGPad<G>;                   // q-heads per anchor row in LDS (padded)
  constexpr int NB = HLM ? 1 : (4 * G + 15) / 16;  // 16-wide blocks of (q-head, group) pairs
  constexpr int BR = HLM ? GP : 4 * NB;          // floats per wave row (q-heads >= G read as 0)
  constexpr bool QSPLIT = DT == ANCHORKV_F32 && !HLM;   // f32 queries enter the key MFMA as bf16 hi + lo
  constexpr int QH = QSPLIT ? 2 : 1;
  extern __shared__ __align__(16) float sm[];
  const int A = a.A;
  const DecLds L = dec_lds(G, A, DT == ANCHORKV_F32, NW, CD);
  uint8_t* smb = reinterpret_cast<uint8_t*>(sm);
  // w[g][a] in fixed point, q-head-major (random anchors spread over the banks)
  unsigned long long* wi = reinterpret_cast<unsigned long long*>(smb);
  float* S = reinterpret_cast<float*>(smb + L.S);         // [A][GP]
  float* rows = reinterpret_cast<float*>(smb + L.rows);   // [NW][TT][BR]
  uint4 (*qbs)[64] = reinterpret_cast<uint4 (*)[64]>(smb + L.qbs);
  float2* qcs = reinterpret_cast<float2*>(smb + L.qcs);  // [NB][64]
  __shared__ int cnt[2][NW];       // per wave and tile parity: key-flagged | value-flagged << 16
  __shared__ int offs[2][130];     // first record of each chunk of the range (and of the chunk after)
  __shared__ __align__(16) int tmaxb[3][GP];
  __shared__ int hot_any[3];       // some wave published a tile maximum
  __shared__ __align__(16) float zrow[BR];
  // running maximum per q-head (log2 units), one copy per wave: every wave
  // takes the same decisions from the same tile maxima; kept in LDS rather
  // than registers (it is read twice per tile)
  __shared__ __align__(16) float mrun_s[NW][GP];

  int bid = blockIdx.x;
  const int sp = bid % a.S2; bid /= a.S2;
  const int h = bid % a.H;
  const int u = bid / a.H;
  const int64_t uh = (int64_t)u * a.H + h;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave: uniform
  const int col = lane & 15, kg = lane >> 4;
  float* wrow = rows + wave * TT * BR;   // this wave's rows
  const int c0 = sp * a.cps, c1 = min(a.C, c0 + a.cps);
  const int t_beg = c0 * kTile, t_end = min(a.N, c1 * kTile);
  const int nch = max(0, c1 - c0);
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
        hd->unit_stride != a.stride || hd->off_words != a.off_words || hd->codec != a.codec ||
        (HLM && (hd->signs[0] != a.signs.x || hd->signs[1] != a.signs.y || hd->signs[2] != a.signs.z ||
                 hd->signs[3] != a.signs.w))) {
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

  // q of this head as floats in LDS ([G][D], in the rows region, free until the first tile)
  float* qf = rows;
  for (int i = threadIdx.x; i < G * D; i += blockDim.x) qf[i] = Elem<DT>::f(q[i]);
  for (int i = threadIdx.x; i < G * A; i += blockDim.x) wi[i] = 0ull;
  if (threadIdx.x < BR) zrow[threadIdx.x] = 0.0f;
  if (threadIdx.x < 3 * GP) (&tmaxb[0][0])[threadIdx.x] = kKeyNegInf;
  if (threadIdx.x < 3) hot_any[threadIdx.x] = 0;
  if (threadIdx.x < NW * GP) (&mrun_s[0][0])[threadIdx.x] = -INFINITY;
  {
    // end of the key records and of the value records: with a joint ranking
    // the key records end where the value records start (the value chunk
    // offsets count from the start of the one record section)
    const int* chk = reinterpret_cast<const int*>(base + a.off_ck);
    const int* chv = reinterpret_cast<const int*>(base + a.off_cv);
    const int kend = a.joint ? chv[0] : a.R_K, vend = a.joint ? a.R_total : a.R_V;
    for (int i = threadIdx.x; i <= nch; i += blockDim.x) {
      const int fl = h * a.C + c0 + i;
      const bool last = fl >= a.H * a.C;
      offs[0][i] = last ? kend : chk[fl];
      offs[1][i] = last ? vend : chv[fl];
    }
  }
  __syncthreads();  // qf, offs

  // code-plane constants: masks (SGPRs) and the exponent bias (one VGPR)
  uint32_t MK[3] = {0x00030003u, 0x000C000Cu, 0x00300030u};
  asm volatile("" : "+s"(MK[0]), "+s"(MK[1]), "+s"(MK[2]));
  // high bit of each code (Hadamard / Lloyd-Max codec): 128 + 2 hi 4^m
  uint32_t MKH[3] = {0x00020002u, 0x00080008u, 0x00200020u};
  if constexpr (HLM) asm volatile("" : "+s"(MKH[0]), "+s"(MKH[1]), "+s"(MKH[2]));
  uint32_t vbias = kCodeBias;
  asm volatile("" : "+v"(vbias));

  // Key-side B fragments: column kappa = 16*cb + col = 4*g + grp; in MFMA step
  // st (= coordinate group st) the lane supplies q[g][d] / 4^m for
  // d = j + 16c, j = 4kg + (e&3), c = 2st + (e>>2), when grp == st, zeros
  // otherwise (exact for bf16 queries: the scale by 4^-m is a power of two).
  // cinit = -128 * (sum of what the column is fed), so the accumulator ends at
  // sum_d q[g][d] code_d.  The same in every wave: wave 0 writes them to LDS,
  // with each column's query sum and initial value.
  if (HLM && wave == 0) {
    // Hadamard / Lloyd-Max codec: rotate the queries once, q' = (1/sqrt(D))
    // H_D diag(s) q (Walsh-Hadamard butterflies: bit 6 of the coordinate
    // inside the lane, bits 0-5 across lanes), then column (q-head g, part)
    // of every step is fed the bf16 hi (part 0) or lo (part 1) piece of q'
    // at all 32 coordinates of the step (scaled by 4^-m like the codes).
    float* qr = qf + G * D;
    for (int g = 0; g < G; ++g) {
      float x0 = sign_of(a.signs, lane) * qf[g * D + lane];
      float x1 = sign_of(a.signs, lane + 64) * qf[g * D + lane + 64];
      const float s0 = x0 + x1, s1 = x0 - x1;
      x0 = s0; x1 = s1;
#pragma unroll
      for (int b = 1; b < 64; b <<= 1) {
        const float o0 = __shfl_xor(x0, b, 64), o1 = __shfl_xor(x1, b, 64);
        x0 = (lane & b) ? o0 - x0 : x0 + o0;
        x1 = (lane & b) ? o1 - x1 : x1 + o1;
      }
      qr[g * D + lane] = x0 * 0.088388347648318f;
      qr[g * D + lane + 64] = x1 * 0.088388347648318f;
    }
    __builtin_amdgcn_wave_barrier();
    const int g = col & 7, part = col >> 3;
    float qs = 0.0f, fed = 0.0f;
    if (g < G)
      for (int d = 0; d < D; ++d) {
        const float x = qr[g * D + d];
        const float xh = bf2f(f2bf(x));
        qs += x;
        fed += (part ? bf2f(f2bf(x - xh)) : xh) * kPlaneInv[plane_of(d >> 4).m];
      }
    qcs[lane] = make_float2(qs, -128.0f * fed);
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      uint16_t v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = 2 * st + (e >> 2);
        const int d = (4 * kg + (e & 3)) + 16 * c;
        const float x = g < G ? qr[g * D + d] : 0.0f;
        const uint16_t xh = f2bf(x);
        const uint16_t xp = part ? f2bf(x - bf2f(xh)) : xh;
        v[e] = f2bf(bf2f(xp) * kPlaneInv[plane_of(c).m]);  // exact: power-of-two scaling
      }
      qbs[st][lane] = make_uint4(v[0] | (uint32_t)v[1] << 16, v[2] | (uint32_t)v[3] << 16,
                                 v[4] | (uint32_t)v[5] << 16, v[6] | (uint32_t)v[7] << 16);
    }
  }
  if (!HLM && wave == 0) {
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
      qcs[cb * 64 + lane] = make_float2(qs, -128.0f * fed);
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
        qbs[(cb * 4 + st) * QH][lane] = make_uint4(vh[0] | (uint32_t)vh[1] << 16, vh[2] | (uint32_t)vh[3] << 16,
                                                   vh[4] | (uint32_t)vh[5] << 16, vh[6] | (uint32_t)vh[7] << 16);
        if constexpr (QSPLIT)
          qbs[(cb * 4 + st) * QH + 1][lane] = make_uint4(vl[0] | (uint32_t)vl[1] << 16, vl[2] | (uint32_t)vl[3] << 16,
                                                         vl[4] | (uint32_t)vl[5] << 16, vl[6] | (uint32_t)vl[7] << 16);
      }
    }
  }
  // value side: B = -128 everywhere cancels the code bias of the A rows
  const bf16x4 bm128_4 = u2_to_frag4(0xC300C300u, 0xC300C300u);

  // pointer words: TPL adjacent tokens' (K word, V word) pairs per lane and
  // tile, loaded two tiles ahead (range-checked: a token past the range reads
  // zero words, so no flags)
  using Words = typename std::conditional<TPL == 1, uint2, uint4>::type;
  const uint32_t* words = reinterpret_cast<const uint32_t*>(base + a.off_words) + (int64_t)h * a.N * 2;
  const __amdgpu_buffer_rsrc_t wrs = buf_rsrc(words + (int64_t)t_beg * 2, (uint32_t)(t_end - t_beg) * 8u);
  auto load_words = [&](int it) -> Words {
    const int off = (int)((uint32_t)(it * kTile + wave * TT + lane * TPL) * 8u);
    if constexpr (TPL == 1) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(wrs, off, 0, 0);
      return make_uint2(v[0], v[1]);
    } else {
      // an odd last token: the 8 bytes past it read as zero only if the whole
      // 16-byte access is out of range, so a 16-byte access that straddles
      // the end is split into two 8-byte loads
      const auto v0 = __builtin_amdgcn_raw_buffer_load_b64(wrs, off, 0, 0);
      const auto v1 = __builtin_amdgcn_raw_buffer_load_b64(wrs, off + 8, 0, 0);
      return make_uint4(v0[0], v0[1], v1[0], v1[1]);
    }
  };
  auto flag_counts = [&](const Words& wv) {
    int nk, nv;
    if constexpr (TPL == 1) {
      nk = __popcll(__ballot((wv.x & 0x8000u) != 0));
      nv = __popcll(__ballot((wv.y & 0x8000u) != 0));
    } else {
      nk = __popcll(__ballot((wv.x & 0x8000u) != 0)) + __popcll(__ballot((wv.z & 0x8000u) != 0));
      nv = __popcll(__ballot((wv.y & 0x8000u) != 0)) + __popcll(__ballot((wv.w & 0x8000u) != 0));
    }
    return nk | (nv << 16);
  };
  Words wq[2];
  wq[0] = load_words(0);
  wq[1] = load_words(1);

  // ---- anchor logits S[a][g] = <q_g, k_a> * c on MFMA, 16 anchors per tile
  // (rows = anchors, K = coordinates, columns = q-heads), while the words load
  {
    using MS = Mfma<DT>;
    const T* AK = reinterpret_cast<const T*>(base + a.off_ak) + (int64_t)h * A * D;
    for (int t = wave; t < (A + 15) / 16; t += NW) {
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
  {
    const int fc = flag_counts(wq[0]);   // flagged counts of tile 0
    if (lane == 0) cnt[0][wave] = fc;
  }
  __syncthreads();  // S, qbs, qcs, cnt[0]; qf is dead (rows become the waves' rows)

  // Record runs of a tile: this wave's key / value records start at the
  // tile's chunk offset plus the counts of the waves before it.
  auto run_of = [&](int it, int par, int& kb, int& nk, int& vb, int& nv) {
    const int ic = min(it, nch);
    // uniform values (every lane reads the same word): the record buffer
    // descriptors built from them then live in scalar registers
    const int mine = __builtin_amdgcn_readfirstlane(cnt[par][wave]);
    const int pre = __builtin_amdgcn_readfirstlane(row_sum_i32(lane < wave ? cnt[par][lane & (NW - 1)] : 0));
    kb = __builtin_amdgcn_readfirstlane(offs[0][ic]) + (pre & 0xFFFF);
    vb = __builtin_amdgcn_readfirstlane(offs[1][ic]) + (pre >> 16);
    nk = it < nch ? (mine & 0xFFFF) : 0;
    nv = it < nch ? (mine >> 16) : 0;
  };
  // bytes of a batch of at most 16 records; the clamp has no scalar
  // instruction, so the result is read back from the first lane to keep the
  // buffer descriptor in scalar registers (a descriptor in vector registers
  // turns every load into a loop over its distinct values)
  auto run_bytes = [](int n) -> uint32_t {
    return (uint32_t)__builtin_amdgcn_readfirstlane(min(max(n, 0), 16) * RB);
  };
  // key batch: lane (col, kg) holds bytes 8kg..8kg+7 of record col and the
  // (scale, zero) words of record col's four groups (Hadamard / Lloyd-Max:
  // the scales of records 4kg + r)
  uint2 kx;
  uint32_t ksz[4];
  auto load_keys = [&](int kb, int nk, uint2& x, uint32_t (&sz)[4]) {
    const __amdgpu_buffer_rsrc_t r = buf_rsrc(recK + (int64_t)kb * RB, run_bytes(nk));
    const auto xx = __builtin_amdgcn_raw_buffer_load_b64(r, col * RB + 8 * kg, 0, 0);
    x = make_uint2(xx[0], xx[1]);
    if constexpr (HLM) {
      // the scale of records 4kg + rr (rows of the Hadamard / Lloyd-Max key MFMA)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) sz[rr] = __builtin_amdgcn_raw_buffer_load_b32(r, (4 * kg + rr) * RB + 32, 0, 0);
    } else {
      // the (scale, zero) words of the four groups of record col
      const uint4 v = buf_load16(r, col * RB + 32);
      sz[0] = v.x; sz[1] = v.y; sz[2] = v.z; sz[3] = v.w;
    }
  };
  // value batch: code word col of records 4kg + e (pairs packed), and the
  // (scale, zero) word of group col & 3 of the same records
  uint32_t vpr[2], vsz[4];
  auto load_values = [&](int vb, int nv, uint32_t (&pr)[2], uint32_t (&sz)[4]) {
    const __amdgpu_buffer_rsrc_t r = buf_rsrc(recV + (int64_t)vb * RB, run_bytes(nv));
#pragma unroll
    for (int e2 = 0; e2 < 2; ++e2) {
      const int r0 = 4 * kg + 2 * e2;
      const uint32_t w0 = __builtin_amdgcn_raw_buffer_load_b16(r, r0 * RB + 2 * col, 0, 0);
      const uint32_t w1 = __builtin_amdgcn_raw_buffer_load_b16(r, (r0 + 1) * RB + 2 * col, 0, 0);
      pr[e2] = w0 | (w1 << 16);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
      sz[e] = __builtin_amdgcn_raw_buffer_load_b32(r, (4 * kg + e) * RB + 32 + (HLM ? 0 : 4 * (col & 3)), 0, 0);
  };
  int kb_cur, nk_cur, vb_cur, nv_cur;
  run_of(0, 0, kb_cur, nk_cur, vb_cur, nv_cur);
  load_keys(kb_cur, nk_cur, kx, ksz);
  load_values(vb_cur, nv_cur, vpr, vsz);

  float* mrun = mrun_s[wave];
  float lacc[G];
#pragma unroll
  for (int g = 0; g < G; ++g) lacc[g] = 0.0f;
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
  // Hadamard / Lloyd-Max value side: the value MFMA rows are the q-heads,
  // q-head g on row 4 (g >> 1) + (g & 1), so that lane (col, kg) holds q-heads
  // 2 kg and 2 kg + 1 (r = 0, 1) of coordinate col + 16 cc, in the rotated
  // coordinates; zh sums p * sigma of the q-head of row col
  float vh[HLM ? 8 : 1][2];
#pragma unroll
  for (int cc = 0; cc < (HLM ? 8 : 1); ++cc)
#pragma unroll
    for (int r = 0; r < 2; ++r) vh[cc][r] = 0.0f;
  float zh = 0.0f;

  // ---- key-residual logits (log2 units) of records b0 .. b0+15 of the
  // wave's run, from the fragments (x, sz) into the wave's rows [b0, b0 + 16)
  // (row = rank)
  auto kbatch = [&](int b0, uint2 x, const uint32_t (&sz)[4]) {
    const uint32_t xs[3][2] = {{x.x, x.y}, {x.x >> 6, x.y >> 6}, {x.x >> 12, x.y >> 12}};
    if constexpr (HLM) {
      // sums over the codes (c-plane) and over their high bits (hi-plane)
      // of the rotated query, then the level polynomial and the record scale
      const float2 qc = qcs[lane];   // (sum of q' of q-head col & 7, initial accumulator of the column)
      f32x4 cacc = {qc.y, qc.y, qc.y, qc.y}, hacc = cacc;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const Plane p0 = plane_of(2 * st), p1 = plane_of(2 * st + 1);
        const int i0 = p0.sh / 6, i1 = p1.sh / 6;
        const bf16x8 bq = bits_to_frag(qbs[st][lane]);
        cacc = M::mma(u4_to_frag(and_or(xs[i0][0], MK[p0.m], vbias), and_or(xs[i0][1], MK[p0.m], vbias),
                                 and_or(xs[i1][0], MK[p1.m], vbias), and_or(xs[i1][1], MK[p1.m], vbias)),
                      bq, cacc);
        hacc = M::mma(u4_to_frag(and_or(xs[i0][0], MKH[p0.m], vbias), and_or(xs[i0][1], MKH[p0.m], vbias),
                                 and_or(xs[i1][0], MKH[p1.m], vbias), and_or(xs[i1][1], MKH[p1.m], vbias)),
                      bq, hacc);
      }
      const bool wr = col < G;   // column col (hi part) plus column col + 8 (lo part)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ii = b0 + 4 * kg + r;
        const float C = cacc[r] + dpp<kDppRor8>(cacc[r]);
        const float Hh = hacc[r] + dpp<kDppRor8>(hacc[r]);
        const float sg = h2f((uint16_t)(sz[r] & 0xFFFFu));
        const float val = sg * fmaf(kLmAlpha, C, fmaf(kLmBeta, Hh, -kLmL2 * qc.x));
        if (wr) wrow[ii * BR + col] = val * a.c;   // rows past the run: see below
      }
      return;
    }
    // code fragments as the B operand (K-slice of record col), the query
    // fragments as the A operand: the rows are (q-head, group) pairs kappa =
    // 16 cb + 4 kg + r, so a lane's four accumulators are the four groups of
    // one q-head and one record, and the groups' scales and zeros combine in
    // the lane
    bf16x8 bf[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const Plane p0 = plane_of(2 * st), p1 = plane_of(2 * st + 1);
      const int i0 = p0.sh / 6, i1 = p1.sh / 6;
      bf[st] = u4_to_frag(and_or(xs[i0][0], MK[p0.m], vbias), and_or(xs[i0][1], MK[p0.m], vbias),
                          and_or(xs[i1][0], MK[p1.m], vbias), and_or(xs[i1][1], MK[p1.m], vbias));
    }
    float scg[4], zrg[4];   // (scale, zero) of the four groups of record col
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      scg[r] = h2f((uint16_t)(sz[r] & 0xFFFFu));
      zrg[r] = h2f((uint16_t)(sz[r] >> 16));
    }
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
      // (sum of q over the group, initial accumulator) of rows 16 cb + 4 kg + r
      const float4 qa = *reinterpret_cast<const float4*>(&qcs[cb * 64 + 4 * kg]);
      const float4 qb = *reinterpret_cast<const float4*>(&qcs[cb * 64 + 4 * kg + 2]);
      f32x4 cacc = {qa.y, qa.w, qb.y, qb.w};
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        cacc = M::mma(bits_to_frag(qbs[(cb * 4 + st) * QH][lane]), bf[st], cacc);
        if constexpr (QSPLIT) cacc = M::mma(bits_to_frag(qbs[(cb * 4 + st) * QH + 1][lane]), bf[st], cacc);
      }
      const float qsum[4] = {qa.x, qa.z, qb.x, qb.z};
      float val = 0.0f;
#pragma unroll
      for (int r = 0; r < 4; ++r) val = fmaf(scg[r], cacc[r], fmaf(zrg[r], qsum[r], val));
      // rows past the run (record b0 + col >= nk, still below the wave's TT
      // rows since the batch starts below nk) take values no one reads: key
      // logits are read for ranks below nk only, and the value weights and
      // zeros are written over every row the value batches read before they
      // read it
      const int g = 4 * cb + kg;
      if (g < G) wrow[(b0 + col) * BR + g] = val * a.c;
    }
  };
  // ---- value residuals of records b0 .. b0+15 of the wave's run (weights in
  // the wave's rows [b0, b0 + 16), zeros past the run), on the K = 16 MFMA:
  // lane (col, kg) feeds records 4kg .. 4kg + 3 of the batch
  auto vbatch = [&](int b0, const uint32_t (&pr)[2], const uint32_t (&sz)[4]) {
    if constexpr (HLM) {
      // A = p * sigma as bf16 hi + lo (two MFMAs into one accumulator), rows
      // 4 (g >> 1) + (g & 1) for q-head g, the other rows zero; B = the
      // c-plane and the hi-plane of the codes; both start from the bias term
      // -128 * (row sums of A)
      const bool rowq = (col & 3) < 2;
      const int g = 2 * (col >> 2) + (col & 1);
      float ps[4];
      float zs = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float pv = (rowq && g < G) ? wrow[(b0 + 4 * kg + e) * BR + g] : 0.0f;
        ps[e] = pv * h2f((uint16_t)(sz[e] & 0xFFFFu));
        zs += ps[e];
      }
      zh += zs;
      uint32_t hp[2], lp[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const uint32_t hb = bf16_pack(ps[2 * k], ps[2 * k + 1]);
        hp[k] = hb;
        lp[k] = bf16_pack(ps[2 * k] - __uint_as_float(hb << 16), ps[2 * k + 1] - __uint_as_float(hb & 0xFFFF0000u));
      }
      const bf16x4 ah = u2_to_frag4(hp[0], hp[1]), al = u2_to_frag4(lp[0], lp[1]);
      f32x4 zb = mma16k(ah, bm128_4, f32x4{0, 0, 0, 0});
      zb = mma16k(al, bm128_4, zb);
      const uint32_t ps6[2] = {pr[0] >> 6, pr[1] >> 6};
      const uint32_t ps12[2] = {pr[0] >> 12, pr[1] >> 12};
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) {
        const Plane pl = plane_of(cc);
        const uint32_t* src = pl.sh == 0 ? pr : pl.sh == 6 ? ps6 : ps12;
        const bf16x4 bc = u2_to_frag4(and_or(src[0], MK[pl.m], vbias), and_or(src[1], MK[pl.m], vbias));
        const bf16x4 bh = u2_to_frag4(and_or(src[0], MKH[pl.m], vbias), and_or(src[1], MKH[pl.m], vbias));
        f32x4 tc = mma16k(ah, bc, zb);
        tc = mma16k(al, bc, tc);
        f32x4 th = mma16k(ah, bh, zb);
        th = mma16k(al, bh, th);
#pragma unroll
        for (int r = 0; r < 2; ++r) vh[cc][r] = fmaf(kLmAlpha, tc[r], fmaf(kLmBeta, th[r], vh[cc][r]));
      }
      return;
    }
    bf16x4 ahi[NB], alo[NB];
    f32x4 zb[NB];  // -128 * row sums of A: cancels the code bias
#pragma unroll
    for (int rb = 0; rb < NB; ++rb) {
      const int g = (16 * rb + col) >> 2;
      float ps[4];
      float zsum = zt[rb];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float pv = wrow[(b0 + 4 * kg + e) * BR + g];
        ps[e] = pv * h2f((uint16_t)(sz[e] & 0xFFFFu));
        zsum = fmaf(pv, h2f((uint16_t)(sz[e] >> 16)), zsum);
      }
      zt[rb] = zsum;
      uint32_t hp[2], lp[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const uint32_t hb = bf16_pack(ps[2 * k], ps[2 * k + 1]);
        const float d0 = ps[2 * k] - __uint_as_float(hb << 16);
        const float d1 = ps[2 * k + 1] - __uint_as_float(hb & 0xFFFF0000u);
        hp[k] = hb;
        lp[k] = bf16_pack(d0, d1);
      }
      ahi[rb] = u2_to_frag4(hp[0], hp[1]);
      alo[rb] = u2_to_frag4(lp[0], lp[1]);
      zb[rb] = mma16k(ahi[rb], bm128_4, f32x4{0, 0, 0, 0});
      zb[rb] = mma16k(alo[rb], bm128_4, zb[rb]);
    }
    const uint32_t ps6[2] = {pr[0] >> 6, pr[1] >> 6};
    const uint32_t ps12[2] = {pr[0] >> 12, pr[1] >> 12};
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      const Plane pl = plane_of(cc);
      const uint32_t* src = pl.sh == 0 ? pr : pl.sh == 6 ? ps6 : ps12;
      const bf16x4 bfr = u2_to_frag4(and_or(src[0], MK[pl.m], vbias), and_or(src[1], MK[pl.m], vbias));
#pragma unroll
      for (int rb = 0; rb < NB; ++rb) {
        f32x4 t = mma16k(ahi[rb], bfr, zb[rb]);
        t = mma16k(alo[rb], bfr, t);
        vacc[rb][cc] += t[cc >> 1];
      }
    }
  };

  for (int base_it = 0; base_it < nch; base_it += 2) {
#pragma unroll
  for (int slot = 0; slot < 2; ++slot) {
    // no early exit: a tile past the range (odd tile count) has no valid
    // token, no record and no maximum, and every wave still takes its barrier
    const int it = base_it + slot;
    const int tm3 = it % 3;
    const int t0 = t_beg + it * kTile + wave * TT + lane * TPL;   // the lane's first token
    const Words wd = wq[slot];
    const Words wn = wq[slot ^ 1];       // words of tile it + 1 (loaded a tile ago)
    wq[slot] = load_words(it + 2);
    {
      const int fc = flag_counts(wn);    // flagged counts of tile it + 1 (read after this tile's barrier)
      if (lane == 0) cnt[slot ^ 1][wave] = fc;
    }
    // ---- pointer words of the lane's tokens
    uint32_t wk[TPL], wv[TPL];
    if constexpr (TPL == 1) { wk[0] = wd.x; wv[0] = wd.y; }
    else { wk[0] = wd.x; wv[0] = wd.y; wk[1] = wd.z; wv[1] = wd.w; }
    bool valid[TPL], fK[TPL], fV[TPL];
    int rK[TPL], rV[TPL];
    {
      unsigned long long bK[TPL], bV[TPL];
#pragma unroll
      for (int k = 0; k < TPL; ++k) {
        valid[k] = it < nch && t0 + k < t_end;
        fK[k] = (wk[k] & 0x8000u) != 0;
        fV[k] = (wv[k] & 0x8000u) != 0;
        bK[k] = __ballot(fK[k]);
        bV[k] = __ballot(fV[k]);
      }
      // rank of token (lane, k) among the wave's flagged tokens, in token order
      int below_k = 0, below_v = 0;
#pragma unroll
      for (int k = 0; k < TPL; ++k) { below_k += lanes_below(bK[k]); below_v += lanes_below(bV[k]); }
      rK[0] = below_k; rV[0] = below_v;
      if constexpr (TPL == 2) { rK[1] = below_k + (fK[0] ? 1 : 0); rV[1] = below_v + (fV[0] ? 1 : 0); }
    }
    const int nK = nk_cur, nV = nv_cur;

    // ---- key-residual logits of the wave's records, 16 per batch; the first
    // batch was loaded a tile ahead, more are read here
    {
      uint2 x = kx;
      uint32_t sz[4] = {ksz[0], ksz[1], ksz[2], ksz[3]};
      for (int b0 = 0; b0 < nK; b0 += 16) {
        if (b0 > 0) load_keys(kb_cur + b0, nK - b0, x, sz);
        kbatch(b0, x, sz);
      }
    }
    __builtin_amdgcn_wave_barrier();  // the wave's rows written before other lanes read them

    // ---- logits of the lane's tokens (kept in registers across the barrier;
    // recomputing them costs two LDS row reads per token, which at eight
    // q-heads cost more than the registers); tile maximum when one passes
    // m_run + kLazy
    auto logits = [&](int k, float (&s)[G]) {
      float Sv[GP], Rv[GP];
      ldsv<GP>(S + (wk[k] & 0x7FFF) * GP, Sv);
      ldsv<GP>(fK[k] ? wrow + rK[k] * BR : zrow, Rv);
      const float gK = h2f((uint16_t)(wk[k] >> 16));
#pragma unroll
      for (int g = 0; g < G; ++g) s[g] = valid[k] ? fmaf(gK, Sv[g], Rv[g]) : -INFINITY;
    };
    float sk[TPL][G];
    {
      float mv[GP];
      ldsv<GP>(mrun, mv);
      bool hot = false;
      float smax[G];
#pragma unroll
      for (int k = 0; k < TPL; ++k) {
        float (&s)[G] = sk[k];
        logits(k, s);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          smax[g] = k == 0 ? s[g] : fmaxf(smax[g], s[g]);
          hot |= s[g] > mv[g] + kLazy;
        }
      }
      if (__any(hot)) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const int mk = wave_max_i32(fkey(smax[g]));
          if (lane == 0) atomicMax(&tmaxb[tm3][g], mk);
        }
        if (lane == 0) hot_any[tm3] = 1;
      }
    }
    if (threadIdx.x < GP) tmaxb[(it + 1) % 3][threadIdx.x] = kKeyNegInf;  // last read two tiles ago
    if (threadIdx.x == 0) hot_any[(it + 1) % 3] = 0;
    lds_barrier();

    // ---- runs of tile it + 1 (its counts are published); its key records
    // go to the key registers now (this tile's are consumed), its value
    // records after this tile's value batch
    int vb_next, nv_next;
    {
      int kb2, nk2;
      run_of(it + 1, slot ^ 1, kb2, nk2, vb_next, nv_next);
      load_keys(kb2, nk2, kx, ksz);
      kb_cur = kb2;
      nk_cur = nk2;
    }
    // ---- lazy rescale (every thread takes the same decision); skipped
    // unless some wave published a tile maximum
    float m_run[GP];
    ldsv<GP>(mrun, m_run);
    if (__builtin_amdgcn_readfirstlane(hot_any[tm3])) {
      bool any = false;
      float fct[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float tm = fkey_inv(tmaxb[tm3][g]);
        fct[g] = 1.0f;
        if (tm > m_run[g] + kLazy) {
          fct[g] = (m_run[g] == -INFINITY) ? 0.0f : exp2_fast(m_run[g] - tm);
          m_run[g] = tm;
          any = true;
        }
      }
      if (any) {
        __builtin_amdgcn_wave_barrier();
        if (lane < G) {
          float mn = 0.0f;
#pragma unroll
          for (int g = 0; g < G; ++g) mn = (g == lane) ? m_run[g] : mn;
          mrun[lane] = mn;
        }
#pragma unroll
        for (int g = 0; g < G; ++g) lacc[g] *= fct[g];
#pragma unroll
        for (int g = 0; g < G; ++g)
          if (fct[g] != 1.0f)
            for (int i = threadIdx.x; i < A; i += blockDim.x)
              wi[g * A + i] = (unsigned long long)__double2ll_rn((double)(long long)wi[g * A + i] * (double)fct[g]);
        if constexpr (HLM) {
#pragma unroll
          for (int r = 0; r < 2; ++r) {
            const int g = 2 * kg + r;
            float f = 1.0f;
#pragma unroll
            for (int gg = 0; gg < G; ++gg) f = (gg == g) ? fct[gg] : f;
#pragma unroll
            for (int cc = 0; cc < 8; ++cc) vh[cc][r] *= f;
          }
          const int gz = 2 * (col >> 2) + (col & 1);   // q-head of row col
          float fz = 1.0f;
#pragma unroll
          for (int gg = 0; gg < G; ++gg) fz = (gg == gz) ? fct[gg] : fz;
          zh *= fz;
        }
#pragma unroll
        for (int rb = 0; rb < (HLM ? 0 : NB); ++rb) {
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
        lds_barrier();
      }
    }
    // ---- softmax weights, w scatter, weights of value-flagged tokens into the
    // wave's rows (zeros after them up to the next multiple of 16).
    // p <= 2 (lazy rescale), so gamma in [0, 8) keeps y = p*gamma*2^38 in
    // [0, 2^42): one f64 fma adds 1.5*2^52, which rounds y to the nearest
    // integer and leaves it in the low 51 bits (p and gamma are exact in f64).
    bool fast = true;
#pragma unroll
    for (int k = 0; k < TPL; ++k) {
      const float gV = h2f((uint16_t)(wv[k] >> 16));
      fast = fast && (!valid[k] || (gV >= 0.0f && gV < 8.0f));
    }
    fast = __all(fast);
    // every token's logits were read from the rows before any value row is
    // written over them (the rows of key logits and of value weights are the
    // same wave-private rows)
    float pk[TPL][BR];
#pragma unroll
    for (int k = 0; k < TPL; ++k) {
      const float (&s)[G] = sk[k];
#pragma unroll
      for (int g = 0; g < BR; ++g) pk[k][g] = 0.0f;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        pk[k][g] = exp2_fast(s[g] - m_run[g]);   // 0 for a token past the range
        lacc[g] += pk[k][g];
      }
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int k = 0; k < TPL; ++k) {
      const int aV = wv[k] & 0x7FFF;
      const float gV = h2f((uint16_t)(wv[k] >> 16));
      if (fast) {
        const double gd = (double)gV * kFxScaleD;
#pragma unroll
        for (int g = 0; g < G; ++g)
          atomicAdd(wi + g * A + aV,
                    (unsigned long long)__double_as_longlong(fma((double)pk[k][g], gd, kRoundMagic)) & kMagicMask);
      } else {
        const float gs = gV * kFxScale;
#pragma unroll
        for (int g = 0; g < G; ++g) atomicAdd(wi + g * A + aV, fx_general(pk[k][g] * gs));
      }
      if (fV[k]) stsv<BR>(wrow + rV[k] * BR, pk[k]);
    }
    {
      float z0[BR];
#pragma unroll
      for (int g = 0; g < BR; ++g) z0[g] = 0.0f;
      const int zr = nV + lane;
      if (zr < ((nV + 15) & ~15)) stsv<BR>(wrow + zr * BR, z0);
    }
    __builtin_amdgcn_wave_barrier();

    // ---- value residuals of the wave's records, 16 per batch (the first
    // batch loaded a tile ahead, more read here)
    {
      uint32_t pr[2] = {vpr[0], vpr[1]};
      uint32_t sz[4] = {vsz[0], vsz[1], vsz[2], vsz[3]};
      for (int b0 = 0; b0 < nV; b0 += 16) {
        if (b0 > 0) load_values(vb_cur + b0, nV - b0, pr, sz);
        vbatch(b0, pr, sz);
      }
    }
    load_values(vb_next, nv_next, vpr, vsz);
    vb_cur = vb_next;
    nv_cur = nv_next;
  }
  }

  // ---- epilogue.  w V on MFMA: wave w takes coordinates 16 (w & 7) .. + 15
  // and, with 16 waves, every other K-step of anchors from (w >> 3); rows =
  // q-heads, K = anchors, columns = coordinates; w in bf16 hi + lo for bf16 data
  __syncthreads();  // every scatter into w done
  static_assert(D == 128 && (NW == 8 || NW == 16), "eight 16-coordinate blocks");
  constexpr int NPART = NW / 8;
  const int part = wave >> 3;
  const int d = 16 * (wave & 7) + col;
  f32x4 ov = {0, 0, 0, 0};
  {
    using MV = Mfma<DT>;
    const T* AV = reinterpret_cast<const T*>(base + a.off_av) + (int64_t)h * A * D;
    for (int a0 = part * MV::KSTEP; a0 < A; a0 += NPART * MV::KSTEP) {
      const int ab = a0 + kg * MV::KW;
      if constexpr (DT == ANCHORKV_BF16) {
        float wvv[8];
        uint32_t vb[4];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          wvv[e] = (col < G && ab + e < A) ? (float)((double)(long long)wi[col * A + ab + e] * kFxInv) : 0.0f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t v0 = ab + 2 * k < A ? (uint32_t)AV[(int64_t)(ab + 2 * k) * D + d] : 0u;
          const uint32_t v1 = ab + 2 * k + 1 < A ? (uint32_t)AV[(int64_t)(ab + 2 * k + 1) * D + d] : 0u;
          vb[k] = v0 | (v1 << 16);
        }
        uint32_t hp[4], lp[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          hp[k] = bf16_pack(wvv[2 * k], wvv[2 * k + 1]);
          lp[k] = bf16_pack(wvv[2 * k] - __uint_as_float(hp[k] << 16), wvv[2 * k + 1] - __uint_as_float(hp[k] & 0xFFFF0000u));
        }
        const bf16x8 bv = u4_to_frag(vb[0], vb[1], vb[2], vb[3]);
        ov = MV::mma(u4_to_frag(hp[0], hp[1], hp[2], hp[3]), bv, ov);
        ov = MV::mma(u4_to_frag(lp[0], lp[1], lp[2], lp[3]), bv, ov);
      } else {
        const float wvv = (col < G && ab < A) ? (float)((double)(long long)wi[col * A + ab] * kFxInv) : 0.0f;
        const float vv = ab < A ? Elem<DT>::f(AV[(int64_t)ab * D + d]) : 0.0f;
        ov = MV::mma(wvv, vv, ov);
      }
    }
  }
  float lw[G];
#pragma unroll
  for (int g = 0; g < G; ++g) lw[g] = wave_sum(lacc[g]);
  __syncthreads();  // w, S and the rows are no longer read: the region holds the partials
  float* pv = reinterpret_cast<float*>(smb + L.pv);    // [NW][G][D]
  float* pwv = reinterpret_cast<float*>(smb + L.pwv);  // [NPART][G][D]
  float* pz = reinterpret_cast<float*>(smb + L.pz);    // [NW][4 BR]: (q-head, group) = 4g + grp
  float* pl = reinterpret_cast<float*>(smb + L.pl);    // [NW][GP]
  if constexpr (HLM) {
    // q-heads 2 kg + r (r = 0, 1) at coordinate col + 16 cc, in the rotated coordinates
#pragma unroll
    for (int cc = 0; cc < 8; ++cc)
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int gq = 2 * kg + r;
        if (gq < G) pv[(wave * G + gq) * D + col + 16 * cc] = vh[cc][r] * kPlaneInv[plane_of(cc).m];
      }
    float z = zh;
    z += __shfl_xor(z, 16, 64);
    z += __shfl_xor(z, 32, 64);
    const int gz = 2 * (col >> 2) + (col & 1);
    if (kg == 0 && (col & 3) < 2 && gz < G) pz[wave * 4 * BR + gz] = z;
  }
#pragma unroll
  for (int rb = 0; rb < (HLM ? 0 : NB); ++rb) {
    // lane (col, kg) of column block cc holds q-head 4rb + kg, coordinate col + 16cc
    const int gq = 4 * rb + kg;
    if (gq < G)
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) pv[(wave * G + gq) * D + col + 16 * cc] = vacc[rb][cc] * kPlaneInv[plane_of(cc).m];
    float z = zt[rb];
    z += __shfl_xor(z, 16, 64);
    z += __shfl_xor(z, 32, 64);
    if (kg == 0) pz[wave * 4 * BR + 16 * rb + col] = z;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int g = 4 * kg + r;
    if (g < G) pwv[(part * G + g) * D + d] = ov[r];
  }
#pragma unroll
  for (int g = 0; g < G; ++g)
    if (lane == g) pl[wave * GP + g] = lw[g];
  __syncthreads();
  float* prot = reinterpret_cast<float*>(smb + L.prot);  // [G][D] (Hadamard / Lloyd-Max codec)
  if constexpr (HLM) {
    // residual part in the rotated coordinates: the waves' partials in a
    // fixed order, minus l2 * sum of p * sigma (the constant term of the levels)
    for (int i = threadIdx.x; i < G * D; i += blockDim.x) {
      const int g = i / D, dd = i % D;
      float r = 0.0f, z = 0.0f;
#pragma unroll 4
      for (int w2 = 0; w2 < NW; ++w2) {
        r += pv[(w2 * G + g) * D + dd];
        z += pz[w2 * 4 * BR + g];
      }
      prot[i] = fmaf(-kLmL2, z, r);
    }
    __syncthreads();
  }
  // thread (q-head, coordinate): the waves' partials in a fixed order
  const int64_t ps = uh * a.S2 + sp;
  for (int i = threadIdx.x; i < G * D; i += blockDim.x) {
    const int g = i / D, dd = i % D;
    float val = 0.0f;
#pragma unroll
    for (int pp = 0; pp < NPART; ++pp) val += pwv[(pp * G + g) * D + dd];
    float l = 0.0f;
    if constexpr (HLM) {
      // back to the input coordinates: diag(s) (1/sqrt(D)) H_D applied to the rotated sum
      float acc = 0.0f;
      for (int k = 0; k < D; ++k) {
        const float x = prot[g * D + k];
        acc += (__popc((unsigned)(dd & k)) & 1) ? -x : x;
      }
      val = fmaf(sign_of(a.signs, dd) * 0.088388347648318f, acc, val);
#pragma unroll 4
      for (int w2 = 0; w2 < NW; ++w2) l += pl[w2 * GP + g];
    } else {
#pragma unroll 4
      for (int w2 = 0; w2 < NW; ++w2) {
        val += pv[(w2 * G + g) * D + dd] + pz[w2 * 4 * BR + 4 * g + dd / 32];
        l += pl[w2 * GP + g];
      }
    }
    const float m = mrun_s[0][g];
    if (a.S2 == 1 && !a.force_part) {
      a.o[(uh * G + g) * D + dd] = val / l;
    } else {
      // several ranges per head, or a tail to follow: publish this one (merged by k_dec_merge)
      a.part_acc[(ps * G + g) * D + dd] = val;
      if (dd == 0) a.part_ml[ps * G + g] = make_float2(m, l);
    }
  }
}

// ------------------------------------------------------------ pre-RoPE keys
// Decode attention over a cache whose keys were stored before the rotary
// embedding (Pith review of AnchorKV, "Assumptions & free parameters": R_t is
// a per-position orthogonal map, so R_t k^_t = gamma R_t k_a + R_t r~_t;
// "Referee Report": RoPE distributes over the decomposition).  The rotation
// depends on each token's position, so the anchor-logit table of the stream
// kernel does not apply: keys are rebuilt and rotated tile by tile in
// registers (the fused-decoder idea of the AnchorKV-adapted page, "Adaptation
// notes"; the layout here is our own) and values rebuilt into LDS.  One
// workgroup of four waves per (unit, head, range of 1024-token chunks), tiles
// of 64 tokens:
//  * wave 0 reads the tile's pointer words, forms the residual-flag masks and
//    the record index of the tile's first flagged token per side, and
//    e^{i t0 theta_p} of the tile's first position for the 64 frequencies
//    (double precision);
//  * wave w rebuilds keys 16w..16w+15 in MFMA A-operand layout: lane (token,
//    kg) holds coordinates 32 st + 8 kg + e (st = 0..3), so the pair (p, p +
//    64) of a rotation sits in one lane; pair p turns by e^{i t0 theta_p}
//    e^{i j theta_p} (j = t - t0, the second factor from a table built once
//    per workgroup); logits against the q-heads on MFMA with the key as bf16
//    hi + lo (the query exact bf16, or hi + lo for f32 caches);
//  * every thread rebuilds a quarter of one value row (bf16 hi + lo planes in LDS);
//  * softmax per q-head by one wave (running maximum, exact rescale);
//  * p v on MFMA: rows q-heads (p as hi + lo), K = 32 tokens, columns 16
//    coordinates (v as hi + lo), three products per block.
// Partials (max, sum, unnormalised output) go to k_dec_merge as the stream
// kernel's do.
template <int DT>
__global__ __launch_bounds__(256) void k_dec_rope(DecArgs a) {
  using T = typename Elem<DT>::T;
  using M = Mfma<ANCHORKV_BF16>;
  constexpr int D = kHeadDim, TT = 64, P = D / 2;
  constexpr int EPC = 16 / (int)sizeof(T);    // elements per 16-byte load
  // rows padded so that the 16 tokens (or q-heads) of one MFMA operand read
  // fall on different LDS banks
  __shared__ __align__(16) float2 ftab[TT][P + 2];   // e^{i j theta_p}, j < 64
  __shared__ __align__(16) float2 e0[P];             // e^{i t0 theta_p} of the tile
  __shared__ __align__(16) uint16_t vh[TT][D + 8];   // rebuilt value rows, bf16 hi
  __shared__ __align__(16) uint16_t vl[TT][D + 8];   // and lo
  __shared__ __align__(16) float ps[16][TT + 4];     // logits, then p (rows >= G stay zero)
  __shared__ uint2 wds[TT];                          // the tile's pointer words (K, V)
  __shared__ unsigned long long fmask[2];            // residual flags of the tile's tokens per side
  __shared__ int rbase[2];                           // record of the tile's first flagged token per side
  __shared__ float fr[kMaxG], mrun[kMaxG], lrun[kMaxG];

  const int G = a.G;
  int bid = blockIdx.x;
  const int sp = bid % a.S2; bid /= a.S2;
  const int h = bid % a.H;
  const int u = bid / a.H;
  const int64_t uh = (int64_t)u * a.H + h;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, kg = lane >> 4;
  const int c0 = sp * a.cps, c1 = min(a.C, c0 + a.cps);
  const int t_beg = c0 * kTile, t_end = min(a.N, c1 * kTile);
  const uint8_t* base = a.cache + (int64_t)u * a.stride;
  const uint8_t* recK = base + a.off_rk;
  const uint8_t* recV = base + a.off_rv;
  const T* AK = reinterpret_cast<const T*>(base + a.off_ak) + (int64_t)h * a.A * D;
  const T* AV = reinterpret_cast<const T*>(base + a.off_av) + (int64_t)h * a.A * D;
  const uint32_t* words = reinterpret_cast<const uint32_t*>(base + a.off_words) + (int64_t)h * a.N * 2;
  const int* chk = reinterpret_cast<const int*>(base + a.off_ck) + h * a.C;
  const int* chv = reinterpret_cast<const int*>(base + a.off_cv) + h * a.C;
  const T* qp = reinterpret_cast<const T*>(a.q) + uh * G * D;

  // the unit's header must describe the plan's cache (see k_dec_stream)
  {
    const UnitHeader* hd = reinterpret_cast<const UnitHeader*>(base);
    if (hd->magic != kMagic || hd->H != a.H || hd->N != a.N || hd->A != a.A || hd->R_K != a.R_K ||
        hd->R_V != a.R_V || hd->unit_stride != a.stride || hd->off_words != a.off_words || hd->codec != a.codec ||
        hd->rope != 1 || hd->rope_theta != a.rope_theta) {
      const float nan = __builtin_nanf("");
      if (a.S2 == 1 && !a.force_part) {
        for (int i = tid; i < G * D; i += 256) a.o[uh * G * D + i] = nan;
      } else {
        const int64_t slot = uh * a.S2 + sp;
        for (int i = tid; i < G * D; i += 256) a.part_acc[slot * G * D + i] = nan;
        if (tid < G) a.part_ml[slot * G + tid] = make_float2(nan, nan);
      }
      return;
    }
  }

  // query fragments (B operand: column = q-head, the lane's K-slice of each
  // 32-coordinate step); f32 queries as bf16 hi + lo
  bf16x8 qb[4], qbl[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = col < G ? Elem<DT>::f(qp[col * D + 32 * st + 8 * kg + e]) : 0.0f;
    split8(x, qb[st], qbl[st]);
  }
  // theta of frequency lane (every thread of a column of ftab has the same
  // one: 256 is a multiple of P); e^{i j theta_p} for j < 64 in double
  // precision, rounded once
  const double theta_l = pow((double)a.rope_theta, -2.0 * lane / D);
  for (int j = tid / P; j < TT; j += 256 / P) {
    double sn, cn;
    sincos((double)j * theta_l, &sn, &cn);
    ftab[j][lane] = make_float2((float)cn, (float)sn);
  }
  for (int i = tid; i < 16 * (TT + 4); i += 256) (&ps[0][0])[i] = 0.0f;
  if (tid < kMaxG) { mrun[tid] = -INFINITY; lrun[tid] = 0.0f; }
  int run_k = 0, run_v = 0;   // wave 0: flagged tokens of the current chunk before the tile
  f32x4 oacc[2] = {f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}};

  // wave 0 holds the next tile's pointer words and e^{i t0 theta} in
  // registers: the words are loaded a tile ahead, the phase advances by
  // e^{i 64 theta} per tile and is recomputed exactly at every 1024-token chunk
  uint2 wd_n = make_uint2(0u, 0u);
  float2 e0_n = make_float2(1.0f, 0.0f), p64 = make_float2(1.0f, 0.0f);
  if (wave == 0) {
    double sn, cn;
    sincos(64.0 * theta_l, &sn, &cn);
    p64 = make_float2((float)cn, (float)sn);
    if (t_beg + lane < t_end) wd_n = *reinterpret_cast<const uint2*>(words + (int64_t)(t_beg + lane) * 2);
    sincos((double)t_beg * theta_l, &sn, &cn);
    e0_n = make_float2((float)cn, (float)sn);
  }

  for (int t0 = t_beg; t0 < t_end; t0 += TT) {
    // ---- wave 0: publish the tile's words, flags, record bases and phase,
    // then start on the next tile's
    if (wave == 0) {
      if ((t0 & (kTile - 1)) == 0) { run_k = 0; run_v = 0; }
      const uint2 wd = wd_n;
      wds[lane] = wd;
      const unsigned long long mk = __ballot((wd.x & 0x8000u) != 0);
      const unsigned long long mv = __ballot((wd.y & 0x8000u) != 0);
      if (lane == 0) {
        const int c = t0 / kTile;
        fmask[0] = mk; fmask[1] = mv;
        rbase[0] = chk[c] + run_k;
        rbase[1] = chv[c] + run_v;
      }
      run_k += __popcll(mk);
      run_v += __popcll(mv);
      e0[lane] = e0_n;
      const int t1 = t0 + TT;
      wd_n = make_uint2(0u, 0u);
      if (t1 + lane < t_end) wd_n = *reinterpret_cast<const uint2*>(words + (int64_t)(t1 + lane) * 2);
      if ((t1 & (kTile - 1)) == 0) {
        double sn, cn;
        sincos((double)t1 * theta_l, &sn, &cn);
        e0_n = make_float2((float)cn, (float)sn);
      } else {
        e0_n = make_float2(e0_n.x * p64.x - e0_n.y * p64.y, e0_n.x * p64.y + e0_n.y * p64.x);
      }
    }
    __syncthreads();

    // ---- every gather of the tile first (anchor rows and records of the
    // key and the value side), then the arithmetic
    const int j = 16 * wave + col;               // key side: this lane's token
    const uint32_t wk = wds[j].x;
    const int r = tid >> 2, qq = tid & 3;        // value side: token r, coordinates 32 qq .. + 31
    const uint32_t wv = wds[r].y;
    uint4 kraw[4][8 / EPC], vraw[32 / EPC];
    {
      const T* ar = AK + (int64_t)(wk & 0x7FFF) * D;
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int i = 0; i < 8 / EPC; ++i) kraw[st][i] = *reinterpret_cast<const uint4*>(ar + 32 * st + 8 * kg + EPC * i);
      const T* vr = AV + (int64_t)(wv & 0x7FFF) * D + 32 * qq;
#pragma unroll
      for (int i = 0; i < 32 / EPC; ++i) vraw[i] = *reinterpret_cast<const uint4*>(vr + EPC * i);
    }
    // key record: code words 8 (kg & 1) .. + 7 (coordinates 32 st + 8 kg + e
    // lie in code word 8 (kg & 1) + e, plane 2 st + kg / 2) and the four
    // (scale, zero) words; value record: all 16 code words and the (scale,
    // zero) of group qq
    uint4 kcw = make_uint4(0, 0, 0, 0), ksz = make_uint4(0, 0, 0, 0), vc01 = kcw, vc23 = kcw;
    uint32_t vsz = 0;
    if (wk & 0x8000u) {
      const uint8_t* rp = recK + (int64_t)(rbase[0] + __popcll(fmask[0] & ((1ull << j) - 1ull))) * kRecBytes;
      kcw = *reinterpret_cast<const uint4*>(rp + 16 * (kg & 1));
      ksz = *reinterpret_cast<const uint4*>(rp + 32);
    }
    if (wv & 0x8000u) {
      const uint8_t* rp = recV + (int64_t)(rbase[1] + __popcll(fmask[1] & ((1ull << r) - 1ull))) * kRecBytes;
      vc01 = *reinterpret_cast<const uint4*>(rp);
      vc23 = *reinterpret_cast<const uint4*>(rp + 16);
      vsz = *reinterpret_cast<const uint32_t*>(rp + 32 + 4 * qq);
    }

    // ---- keys of wave w's 16 tokens: rebuild, rotate, logits on MFMA
    {
      const float gk = h2f((uint16_t)(wk >> 16));
      float x[4][8];
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int i = 0; i < 8 / EPC; ++i) {
          T v[EPC];
          *reinterpret_cast<uint4*>(v) = kraw[st][i];
#pragma unroll
          for (int e = 0; e < EPC; ++e) x[st][EPC * i + e] = gk * Elem<DT>::f(v[e]);
        }
      if (wk & 0x8000u) {
        const uint32_t cws[4] = {kcw.x, kcw.y, kcw.z, kcw.w};
        const uint32_t szs[4] = {ksz.x, ksz.y, ksz.z, ksz.w};
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const float sc = h2f((uint16_t)(szs[st] & 0xFFFFu)), zr = h2f((uint16_t)(szs[st] >> 16));
          const int sh = 2 * (2 * st + (kg >> 1));
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t code = ((cws[e >> 1] >> (16 * (e & 1) + sh)) & 3u);
            x[st][e] += fmaf(sc, (float)code, zr);
          }
        }
      }
      // pair p = 32 st + 8 kg + e (st = 0, 1) with p + 64: turn by t theta_p
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int pp = 32 * st + 8 * kg + e;
          const float2 a0 = e0[pp], b0 = ftab[j][pp];
          const float cs = a0.x * b0.x - a0.y * b0.y, sn = a0.x * b0.y + a0.y * b0.x;
          const float x0 = x[st][e], x1 = x[st + 2][e];
          x[st][e] = x0 * cs - x1 * sn;
          x[st + 2][e] = x0 * sn + x1 * cs;
        }
      f32x4 acc = {0, 0, 0, 0};
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        bf16x8 kh, kl;
        split8(x[st], kh, kl);
        acc = M::mma(kh, qb[st], acc);
        acc = M::mma(kl, qb[st], acc);
        if constexpr (DT == ANCHORKV_F32) acc = M::mma(kh, qbl[st], acc);
      }
      if (col < G)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int jr = 16 * wave + 4 * kg + rr;
          ps[col][jr] = t0 + jr < t_end ? acc[rr] * a.c : -INFINITY;
        }
    }
    // ---- values: thread (token r, quarter qq) rebuilds coordinates 32 qq .. + 31
    {
      const float gv = h2f((uint16_t)(wv >> 16));
      float v[32];
#pragma unroll
      for (int i = 0; i < 32 / EPC; ++i) {
        T xx[EPC];
        *reinterpret_cast<uint4*>(xx) = vraw[i];
#pragma unroll
        for (int e = 0; e < EPC; ++e) v[EPC * i + e] = gv * Elem<DT>::f(xx[e]);
      }
      if (wv & 0x8000u) {
        // coordinate 32 qq + e: code word e & 15, plane 2 qq + e / 16; group qq
        const uint32_t cw[8] = {vc01.x, vc01.y, vc01.z, vc01.w, vc23.x, vc23.y, vc23.z, vc23.w};
        const float sc = h2f((uint16_t)(vsz & 0xFFFFu)), zr = h2f((uint16_t)(vsz >> 16));
#pragma unroll
        for (int e = 0; e < 32; ++e) {
          const int jw = e & 15, sh = 2 * (2 * qq + (e >> 4));
          const uint32_t code = (cw[jw >> 1] >> (16 * (jw & 1) + sh)) & 3u;
          v[e] += fmaf(sc, (float)code, zr);
        }
      }
      if (t0 + r >= t_end)
#pragma unroll
        for (int e = 0; e < 32; ++e) v[e] = 0.0f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        bf16x8 hi, lo;
        split8(v + 8 * k, hi, lo);
        *reinterpret_cast<bf16x8*>(&vh[r][32 * qq + 8 * k]) = hi;
        *reinterpret_cast<bf16x8*>(&vl[r][32 * qq + 8 * k]) = lo;
      }
    }
    __syncthreads();
    // ---- softmax per q-head: wave w takes q-heads w, w + 4
    for (int g = wave; g < G; g += 4) {
      const float x = ps[g][lane];
      const float mn = fmaxf(mrun[g], wave_max(x));
      const float f = mrun[g] == -INFINITY ? 0.0f : exp2_fast(mrun[g] - mn);
      const float p = x == -INFINITY ? 0.0f : exp2_fast(x - mn);
      ps[g][lane] = p;
      const float sum = wave_sum(p);
      if (lane == 0) { fr[g] = f; lrun[g] = fmaf(lrun[g], f, sum); mrun[g] = mn; }
    }
    __syncthreads();
    // ---- p v: wave w owns coordinate blocks 2w, 2w + 1
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
        uint32_t wh[4], wl[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r0 = ks * 32 + kg * 8 + 2 * e;
          wh[e] = (uint32_t)vh[r0][d] | ((uint32_t)vh[r0 + 1][d] << 16);
          wl[e] = (uint32_t)vl[r0][d] | ((uint32_t)vl[r0 + 1][d] << 16);
        }
        const bf16x8 vbh = bits_to_frag(make_uint4(wh[0], wh[1], wh[2], wh[3]));
        const bf16x8 vbl = bits_to_frag(make_uint4(wl[0], wl[1], wl[2], wl[3]));
        oacc[b] = M::mma(ph, vbh, oacc[b]);
        oacc[b] = M::mma(pl, vbh, oacc[b]);
        oacc[b] = M::mma(ph, vbl, oacc[b]);
      }
    }
    __syncthreads();   // words, e0, value rows, ps and fr are rewritten by the next tile
  }
  const bool part = a.S2 > 1 || a.force_part;
  const int64_t slot = uh * a.S2 + sp;
  if (part && tid < G) a.part_ml[slot * G + tid] = make_float2(mrun[tid], lrun[tid]);
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int g = 4 * kg + r;
      const int d = (2 * wave + b) * 16 + col;
      if (g < G) {
        if (part) a.part_acc[(slot * G + g) * D + d] = oacc[b][r];
        else a.o[(uh * G + g) * D + d] = oacc[b][r] / lrun[g];
      }
    }
}

// ------------------------------------------------ pre-RoPE keys, weight table
// The same decode as k_dec_rope with the value side organised as in the
// stream kernel: o = (w V_anchors) + sum over value-flagged tokens of
// p_t r~^V_t, with w[g][a] = sum over tokens of anchor a of p_t gamma^V_t
// accumulated in LDS in 64-bit fixed point (scale and rounding as in the
// stream kernel), so no value anchor row is gathered per token; only the
// value residuals of flagged tokens are rebuilt (bf16 hi + lo rows, compacted)
// and multiplied on MFMA.  The running maximum is lazy (raised when a tile
// passes it by 2^1), so w is rescaled only then.  Keys as in k_dec_rope, with
// each wave's phases e^{i t theta_p} taken from its first token and a table
// for the 16 tokens after it; a tile's anchor rows and key records are loaded
// a tile ahead.  One workgroup of four waves per (unit, head, range), tiles
// of 64 tokens, two barriers per tile:
//  A. wave w rebuilds, rotates and scores the keys of tokens 16w .. 16w + 15
//     and publishes its tile maxima when they pass the running maximum by 2^1;
//  B. after the first barrier: rescale if a maximum was published; thread
//     (token, q-head quarter) forms p, scatters p gamma^V into w, and writes p
//     of a value-flagged token into its compacted column; the flagged tokens'
//     value residuals are rebuilt into LDS rows;
//  C. after the second barrier: p r~^V on MFMA over the compacted rows.
// Every wave holds the pointer words of the whole tile (one token per lane,
// loaded two tiles ahead), so residual ranks and record offsets come from its
// own ballots.  Used while the [G][A] table fits kRopeWMaxBytes.
constexpr int kRopeWMaxBytes = 64 * 1024;
constexpr int kRopeRows = 32;   // compacted value-residual rows per round

template <int DT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void k_dec_rope_w(DecArgs a) {
  using T = typename Elem<DT>::T;
  using M = Mfma<ANCHORKV_BF16>;
  constexpr int D = kHeadDim, TT = 64, P = D / 2, RR = kRopeRows;
  constexpr int EPC = 16 / (int)sizeof(T);   // elements per 16-byte load
  constexpr int NK = 8 / EPC;                // 16-byte loads per 8 coordinates
  extern __shared__ __align__(16) unsigned long long wi[];   // [G][A] fixed point
  __shared__ __align__(16) float2 ftab[16][P + 2];   // e^{i j theta_p}, j < 16
  __shared__ __align__(16) float2 e0w[4][P];         // e^{i t_w theta_p}, t_w = wave w's first key token
  __shared__ __align__(16) float ps[kMaxG][TT + 4];  // logits (log2 units), one row per q-head
  __shared__ __align__(16) float pc[kMaxG][TT + 4];  // p of the value-flagged tokens, compacted (zeros after)
  __shared__ __align__(16) uint16_t vh[RR][D + 8];   // their value residuals, bf16 hi
  __shared__ __align__(16) uint16_t vl[RR][D + 8];   // and lo
  __shared__ int tmaxb[2][kMaxG];
  __shared__ int hotb[2];
  __shared__ float lsum[4][kMaxG];
  __shared__ __align__(16) uint4 qfr[4][2][64];      // query B fragments per step (bf16 hi, lo)
  __shared__ double thl[P];                          // theta_p
  __shared__ float2 p64s[P];                         // e^{i 64 theta_p}

  const int G = a.G, A = a.A;
  int bid = blockIdx.x;
  const int sp = bid % a.S2; bid /= a.S2;
  const int h = bid % a.H;
  const int u = bid / a.H;
  const int64_t uh = (int64_t)u * a.H + h;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, kg = lane >> 4;
  const int c0 = sp * a.cps, c1 = min(a.C, c0 + a.cps);
  const int t_beg = c0 * kTile, t_end = min(a.N, c1 * kTile);
  const int ntile = max(0, (t_end - t_beg + TT - 1) / TT);
  const uint8_t* base = a.cache + (int64_t)u * a.stride;
  const uint8_t* recK = base + a.off_rk;
  const uint8_t* recV = base + a.off_rv;
  const T* AK = reinterpret_cast<const T*>(base + a.off_ak) + (int64_t)h * A * D;
  const T* AV = reinterpret_cast<const T*>(base + a.off_av) + (int64_t)h * A * D;
  const uint32_t* words = reinterpret_cast<const uint32_t*>(base + a.off_words) + (int64_t)h * a.N * 2;
  const int* chk = reinterpret_cast<const int*>(base + a.off_ck) + h * a.C;
  const int* chv = reinterpret_cast<const int*>(base + a.off_cv) + h * a.C;
  const T* qp = reinterpret_cast<const T*>(a.q) + uh * G * D;

  // the unit's header must describe the plan's cache (see k_dec_stream)
  {
    const UnitHeader* hd = reinterpret_cast<const UnitHeader*>(base);
    if (hd->magic != kMagic || hd->H != a.H || hd->N != a.N || hd->A != A || hd->R_K != a.R_K ||
        hd->R_V != a.R_V || hd->unit_stride != a.stride || hd->off_words != a.off_words || hd->codec != a.codec ||
        hd->rope != 1 || hd->rope_theta != a.rope_theta) {
      const float nan = __builtin_nanf("");
      if (a.S2 == 1 && !a.force_part) {
        for (int i = tid; i < G * D; i += 256) a.o[uh * G * D + i] = nan;
      } else {
        const int64_t slot = uh * a.S2 + sp;
        for (int i = tid; i < G * D; i += 256) a.part_acc[slot * G * D + i] = nan;
        if (tid < G) a.part_ml[slot * G + tid] = make_float2(nan, nan);
      }
      return;
    }
  }

  // query fragments (B operand: column = q-head, the lane's K-slice of each
  // 32-coordinate step) as bf16 hi + lo, in LDS (read per tile, no
  // registers held across the loop); wave w writes step w
  {
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = col < G ? Elem<DT>::f(qp[col * D + 32 * wave + 8 * kg + e]) : 0.0f;
    bf16x8 hi, lo;
    split8(x, hi, lo);
    qfr[wave][0][lane] = __builtin_bit_cast(uint4, hi);
    qfr[wave][1][lane] = __builtin_bit_cast(uint4, lo);
  }
  // lane = frequency p of the wave's phase: theta_p in double precision
  {
    const double theta_l = pow((double)a.rope_theta, -2.0 * lane / D);
    for (int j = wave; j < 16; j += 4) {
      double sn, cn;
      sincos((double)j * theta_l, &sn, &cn);
      ftab[j][lane] = make_float2((float)cn, (float)sn);
    }
    if (wave == 0) {
      double sn, cn;
      sincos(64.0 * theta_l, &sn, &cn);
      thl[lane] = theta_l;
      p64s[lane] = make_float2((float)cn, (float)sn);
    }
  }
  for (int i = tid; i < G * A; i += 256) wi[i] = 0ull;
  for (int i = tid; i < kMaxG * (TT + 4); i += 256) (&pc[0][0])[i] = 0.0f;
  // value rows start as zeros: a row past a tile's flagged count keeps an
  // earlier tile's finite values, multiplied by a zero p
  for (int i = tid; i < RR * (D + 8); i += 256) { (&vh[0][0])[i] = 0; (&vl[0][0])[i] = 0; }
  if (tid < 2 * kMaxG) (&tmaxb[0][0])[tid] = kKeyNegInf;
  if (tid < 2) hotb[tid] = 0;
  float2 e0r = make_float2(1.0f, 0.0f);   // e^{i (t0 + 16 wave) theta_lane} of the current tile

  // pointer words, one token per lane, two tiles ahead (zero past the range)
  const __amdgpu_buffer_rsrc_t wrs = buf_rsrc(words + (int64_t)t_beg * 2, (uint32_t)(t_end - t_beg) * 8u);
  auto load_words = [&](int it) -> uint2 {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(wrs, (int)((uint32_t)(it * TT + lane) * 8u), 0, 0);
    return make_uint2(v[0], v[1]);
  };
  uint2 wd0 = load_words(0), wd1 = load_words(1), wd2;

  // this lane's key token (16 wave + col): anchor row chunks, and its record
  // (code words 8 (kg & 1) .. + 7 and the four (scale, zero) words) when flagged
  uint32_t wk = 0;
  uint4 kraw[4][NK];
  uint4 kcw = make_uint4(0, 0, 0, 0), ksz = kcw;
  // (rank: the token's place among the tile's key-flagged tokens)
  auto load_key = [&](uint32_t w, int rb, int rank) {
    const T* ar = AK + (int64_t)(w & 0x7FFF) * D;
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int i = 0; i < NK; ++i) kraw[st][i] = *reinterpret_cast<const uint4*>(ar + 32 * st + 8 * kg + EPC * i);
    if (w & 0x8000u) {
      const uint8_t* rp = recK + (int64_t)(rb + rank) * kRecBytes;
      kcw = *reinterpret_cast<const uint4*>(rp + 16 * (kg & 1));
      ksz = *reinterpret_cast<const uint4*>(rp + 32);
    }
  };
  // chunk bookkeeping (uniform): flagged tokens of the current chunk before the tile
  int run_k = 0, run_v = 0;
  {
    // lane = token: its rank among the flagged tokens, handed to key lane (col, kg)
    const int rk = lanes_below(__ballot((wd0.x & 0x8000u) != 0));
    wk = __shfl(wd0.x, 16 * wave + col, 64);
    load_key(wk, __builtin_amdgcn_readfirstlane(chk[c0]), __shfl(rk, 16 * wave + col, 64));
  }

  float m_run[kMaxG];
#pragma unroll
  for (int g = 0; g < kMaxG; ++g) m_run[g] = -INFINITY;
  // copies for this thread's q-heads: column col of the key MFMA, and q-heads
  // (lane & 3) + 4 gi of the softmax step (refreshed when m_run changes)
  float m_col = -INFINITY, m_q[2] = {-INFINITY, -INFINITY};
  float lacc[2] = {0.0f, 0.0f};
  f32x4 oacc[2] = {f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}};
  __syncthreads();   // ftab, wi, pc, tmaxb

  for (int it = 0; it < ntile; ++it) {
    const int t0 = t_beg + it * TT;
    const int par = it & 1;
    const int c = t0 / kTile;
    if ((t0 & (kTile - 1)) == 0) { run_k = 0; run_v = 0; }
    const int rbk = __builtin_amdgcn_readfirstlane(chk[c]) + run_k;
    const int rbv = __builtin_amdgcn_readfirstlane(chv[c]) + run_v;
    const unsigned long long kmask = __ballot((wd0.x & 0x8000u) != 0);
    const unsigned long long vmask = __ballot((wd0.y & 0x8000u) != 0);
    const int nfl = __popcll(vmask);
    wd2 = load_words(it + 2);

    // value residual records of this tile's first round of compacted rows:
    // wave rank wr = (wave - tile) mod 4 rebuilds rows 16 wr + (lane >> 2),
    // coordinates 32 (lane & 3) .. + 31 (ranks 0, 1: rows 0..31, the first
    // round; 2, 3: the second), so that with few flagged tokens one wave
    // does the work, a different one from tile to tile
    const int qq = lane & 3;
    const int wr = (wave - it) & 3;
    const int vrow = 16 * wr + (lane >> 2);
    uint4 vc01 = make_uint4(0, 0, 0, 0), vc23 = vc01;
    uint32_t vsz = 0;
    if (wr < 2 && vrow < nfl) {
      const uint8_t* rp = recV + (int64_t)(rbv + vrow) * kRecBytes;
      vc01 = *reinterpret_cast<const uint4*>(rp);
      vc23 = *reinterpret_cast<const uint4*>(rp + 16);
      vsz = *reinterpret_cast<const uint32_t*>(rp + 32 + 4 * qq);
    }

    // ---- A. the wave's phases for this tile, then its 16 keys
    if ((t0 & (kTile - 1)) == 0) {
      double sn, cn;
      sincos((double)(t0 + 16 * wave) * thl[lane], &sn, &cn);
      e0r = make_float2((float)cn, (float)sn);
    } else {
      const float2 p64 = p64s[lane];
      e0r = make_float2(e0r.x * p64.x - e0r.y * p64.y, e0r.x * p64.y + e0r.y * p64.x);
    }
    e0w[wave][lane] = e0r;
    __builtin_amdgcn_wave_barrier();
    {
      const float gk = h2f((uint16_t)(wk >> 16));
      float x[4][8];
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int i = 0; i < NK; ++i) {
          T v[EPC];
          *reinterpret_cast<uint4*>(v) = kraw[st][i];
#pragma unroll
          for (int e = 0; e < EPC; ++e) x[st][EPC * i + e] = gk * Elem<DT>::f(v[e]);
        }
      if (wk & 0x8000u) {
        const uint32_t cws[4] = {kcw.x, kcw.y, kcw.z, kcw.w};
        const uint32_t szs[4] = {ksz.x, ksz.y, ksz.z, ksz.w};
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const float sc = h2f((uint16_t)(szs[st] & 0xFFFFu)), zr = h2f((uint16_t)(szs[st] >> 16));
          const int sh = 2 * (2 * st + (kg >> 1));
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t code = (cws[e >> 1] >> (16 * (e & 1) + sh)) & 3u;
            x[st][e] += fmaf(sc, (float)code, zr);
          }
        }
      }
      // pair p = 32 st + 8 kg + e (st = 0, 1) with p + 64: turn by t theta_p,
      // t = t_w + col
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int pp = 32 * st + 8 * kg + e;
          const float2 a0 = e0w[wave][pp], b0 = ftab[col][pp];
          const float cs = a0.x * b0.x - a0.y * b0.y, sn = a0.x * b0.y + a0.y * b0.x;
          const float x0 = x[st][e], x1 = x[st + 2][e];
          x[st][e] = x0 * cs - x1 * sn;
          x[st + 2][e] = x0 * sn + x1 * cs;
        }
      f32x4 acc = {0, 0, 0, 0};
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        bf16x8 kh, kl;
        split8(x[st], kh, kl);
        const bf16x8 qh = bits_to_frag(qfr[st][0][lane]);
        acc = M::mma(kh, qh, acc);
        acc = M::mma(kl, qh, acc);
        if constexpr (DT == ANCHORKV_F32) acc = M::mma(kh, bits_to_frag(qfr[st][1][lane]), acc);
      }
      // logits of tokens 16 wave + 4 kg + rr for q-head col; the tile maximum
      // of the column, published when it passes the running maximum by 2^1
      float lm = -INFINITY;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int jr = 16 * wave + 4 * kg + rr;
        const float s = t0 + jr < t_end ? acc[rr] * a.c : -INFINITY;
        if (col < G) ps[col][jr] = s;
        lm = fmaxf(lm, s);
      }
      lm = fmaxf(lm, __shfl_xor(lm, 16, 64));
      lm = fmaxf(lm, __shfl_xor(lm, 32, 64));
      const bool hot = col < G && lm > m_col + kLazy;
      if (__any(hot)) {
        if (hot && kg == 0) atomicMax(&tmaxb[par][col], fkey(lm));
        if (lane == 0) hotb[par] = 1;
      }
    }
    // the next tile's key gathers (its words arrived a tile ago)
    {
      const int t1 = t0 + TT;
      const int rbk1 = (t1 & (kTile - 1)) == 0 ? __builtin_amdgcn_readfirstlane(chk[min(c + 1, a.C - 1)])
                                                : rbk + __popcll(kmask);
      const int rk = lanes_below(__ballot((wd1.x & 0x8000u) != 0));
      wk = __shfl(wd1.x, 16 * wave + col, 64);
      kcw = make_uint4(0, 0, 0, 0);
      ksz = kcw;
      load_key(wk, rbk1, __shfl(rk, 16 * wave + col, 64));
    }
    lds_barrier();

    // ---- B. rescale (uniform decision), p, w scatter, compacted rows
    if (__builtin_amdgcn_readfirstlane(hotb[par])) {
      bool any = false;
      float f[kMaxG];
#pragma unroll
      for (int g = 0; g < kMaxG; ++g) {
        f[g] = 1.0f;
        if (g < G) {
          const float tm = fkey_inv(__builtin_amdgcn_readfirstlane(tmaxb[par][g]));
          if (tm > m_run[g] + kLazy) {
            f[g] = m_run[g] == -INFINITY ? 0.0f : exp2_fast(m_run[g] - tm);
            m_run[g] = tm;
            any = true;
          }
        }
      }
      if (any) {
#pragma unroll
        for (int gi = 0; gi < 2; ++gi) {
          float fg = 1.0f, mg = -INFINITY;
#pragma unroll
          for (int g = 0; g < kMaxG; ++g) {
            fg = (g == qq + 4 * gi) ? f[g] : fg;
            mg = (g == qq + 4 * gi) ? m_run[g] : mg;
          }
          lacc[gi] *= fg;
          m_q[gi] = mg;
        }
#pragma unroll
        for (int g = 0; g < kMaxG; ++g) m_col = (g == col) ? m_run[g] : m_col;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          float fg = 1.0f;
#pragma unroll
          for (int g = 0; g < kMaxG; ++g) fg = (g == 4 * kg + rr) ? f[g] : fg;
          oacc[0][rr] *= fg;
          oacc[1][rr] *= fg;
        }
        for (int i = tid; i < G * A; i += 256) {
          const int g = i / A;
          float fg = 1.0f;
#pragma unroll
          for (int gg = 0; gg < kMaxG; ++gg) fg = (gg == g) ? f[gg] : fg;
          if (fg != 1.0f) wi[i] = (unsigned long long)__double2ll_rn((double)(long long)wi[i] * (double)fg);
        }
        lds_barrier();   // every thread takes this branch: w rescaled before any scatter below
      }
    }
    if (tid < kMaxG) tmaxb[par ^ 1][tid] = kKeyNegInf;   // read last in the previous tile
    if (tid == 0) hotb[par ^ 1] = 0;
    {
      // thread (token r, quarter qq): q-heads qq, qq + 4
      const int r = 16 * wave + (lane >> 2);
      const uint32_t wv = __shfl(wd0.y, r, 64);
      const bool valid = t0 + r < t_end;
      const int aV = wv & 0x7FFF;
      const float gV = h2f((uint16_t)(wv >> 16));
      const bool fl = (wv & 0x8000u) != 0;
      const int kr = __shfl(lanes_below(vmask), r, 64);   // rank among the value-flagged tokens
      const bool fast = gV >= 0.0f && gV < 8.0f;
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) {
        const int g = qq + 4 * gi;
        if (g < G && valid) {
          const float p = exp2_fast(ps[g][r] - m_q[gi]);
          lacc[gi] += p;
          const unsigned long long fx =
              fast ? (unsigned long long)__double_as_longlong(fma((double)p, (double)gV * kFxScaleD, kRoundMagic)) &
                         kMagicMask
                   : fx_general(p * gV * kFxScale);
          atomicAdd(wi + g * A + aV, fx);
          if (fl) pc[g][kr] = p;
        }
      }
      // zeros after the compacted columns, up to the rounds' width (thread:
      // q-head tid / 32, column tid % 32 of each round)
      {
        const int g = tid >> 5, k = tid & 31;
        if (g < G) {
          if (k >= nfl) pc[g][k] = 0.0f;
          if (nfl > RR && k + RR >= nfl) pc[g][k + RR] = 0.0f;
        }
      }
    }
    // value residual rows of the first round
    auto rebuild = [&](int slot, const uint4& c01, const uint4& c23, uint32_t sz) {
      float v[32];
      const uint32_t cw[8] = {c01.x, c01.y, c01.z, c01.w, c23.x, c23.y, c23.z, c23.w};
      const float sc = h2f((uint16_t)(sz & 0xFFFFu)), zr = h2f((uint16_t)(sz >> 16));
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const int jw = e & 15, sh = 2 * (2 * qq + (e >> 4));
        const uint32_t code = (cw[jw >> 1] >> (16 * (jw & 1) + sh)) & 3u;
        v[e] = fmaf(sc, (float)code, zr);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        bf16x8 hi, lo;
        split8(v + 8 * k, hi, lo);
        *reinterpret_cast<bf16x8*>(&vh[slot][32 * qq + 8 * k]) = hi;
        *reinterpret_cast<bf16x8*>(&vl[slot][32 * qq + 8 * k]) = lo;
      }
    };
    if (wr < 2 && vrow < nfl) rebuild(vrow, vc01, vc23, vsz);
    lds_barrier();

    // ---- C. p r~ on MFMA: rows q-heads (p as hi + lo), K = 32 compacted
    // tokens, columns 16 coordinates (r~ as hi + lo); wave w owns coordinate
    // blocks 2w, 2w + 1
    auto pv_round = [&](int k0) {
      float p8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) p8[e] = col < G ? pc[col][k0 + 8 * kg + e] : 0.0f;
      bf16x8 ph, pl;
      split8(p8, ph, pl);
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int d = (2 * wave + b) * 16 + col;
        uint32_t wh[4], wl[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r0 = 8 * kg + 2 * e;
          wh[e] = (uint32_t)vh[r0][d] | ((uint32_t)vh[r0 + 1][d] << 16);
          wl[e] = (uint32_t)vl[r0][d] | ((uint32_t)vl[r0 + 1][d] << 16);
        }
        const bf16x8 vbh = bits_to_frag(make_uint4(wh[0], wh[1], wh[2], wh[3]));
        const bf16x8 vbl = bits_to_frag(make_uint4(wl[0], wl[1], wl[2], wl[3]));
        oacc[b] = M::mma(ph, vbh, oacc[b]);
        oacc[b] = M::mma(pl, vbh, oacc[b]);
        oacc[b] = M::mma(ph, vbl, oacc[b]);
      }
    };
    if (nfl > 0) {
      pv_round(0);
      if (nfl > RR) {
        // rare: a second round of rows (every thread takes it: nfl is uniform)
        lds_barrier();   // round-0 rows read
        if (wr >= 2 && vrow < nfl) {
          const int row = vrow;   // 32 .. 63
          const uint8_t* rp = recV + (int64_t)(rbv + row) * kRecBytes;
          const uint4 c01 = *reinterpret_cast<const uint4*>(rp);
          const uint4 c23 = *reinterpret_cast<const uint4*>(rp + 16);
          const uint32_t sz = *reinterpret_cast<const uint32_t*>(rp + 32 + 4 * qq);
          rebuild(row - RR, c01, c23, sz);
        }
        lds_barrier();
        pv_round(RR);
      }
    }
    run_k += __popcll(kmask);
    run_v += nfl;
    wd0 = wd1;
    wd1 = wd2;
  }

  // ---- epilogue: softmax sums, residual part, w V (thread: coordinate d,
  // q-heads gh, gh + 2, gh + 4, gh + 6)
  const int qq = lane & 3;
#pragma unroll
  for (int gi = 0; gi < 2; ++gi) {
    float v = lacc[gi];
    v += __shfl_xor(v, 4, 64);
    v += __shfl_xor(v, 8, 64);
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    const int g = qq + 4 * gi;
    if (lane < 4 && g < G) lsum[wave][g] = v;
  }
  __syncthreads();   // every scatter into w done; vh is free
  float* po = reinterpret_cast<float*>(&vh[0][0]);   // [G][D] residual part
  static_assert(sizeof(vh) >= kMaxG * D * sizeof(float), "residual part fits the rows");
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int g = 4 * kg + rr;
      if (g < G) po[g * D + (2 * wave + b) * 16 + col] = oacc[b][rr];
    }
  __syncthreads();
  const int d = tid & (D - 1), gh = tid >> 7;
  float accv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int aa = 0; aa < A; ++aa) {
    const float v = Elem<DT>::f(AV[(int64_t)aa * D + d]);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int g = gh + 2 * k;
      if (g < G) accv[k] = fmaf((float)((double)(long long)wi[g * A + aa] * kFxInv), v, accv[k]);
    }
  }
  const bool part = a.S2 > 1 || a.force_part;
  const int64_t slot = uh * a.S2 + sp;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int g = gh + 2 * k;
    if (g < G) {
      const float l = (lsum[0][g] + lsum[1][g]) + (lsum[2][g] + lsum[3][g]);
      const float val = accv[k] + po[g * D + d];
      if (part) {
        a.part_acc[(slot * G + g) * D + d] = val;
        if (d == 0) {
          float mg = 0.0f;
#pragma unroll
          for (int gg = 0; gg < kMaxG; ++gg) mg = (gg == g) ? m_run[gg] : mg;
          a.part_ml[slot * G + g] = make_float2(mg, l);
        }
      } else {
        a.o[(uh * G + g) * D + d] = val / l;
      }
    }
  }
}

// Per (unit, head, q-head) with several token ranges (and an optional tail
// partial): o = sum_s f_s acc_s / sum_s f_s l_s with f_s = 2^(m_s - max m).
// One block of 128 threads (one per coordinate) per q-head: the range
// weights f_s are formed once in LDS, then every thread sums its coordinate
// over the ranges in a fixed order with the loads issued together.
constexpr int kMergeMax = 64 + 16;   // compressed ranges (<= 64) + tail ranges (<= 16)
__global__ __launch_bounds__(128) void k_dec_merge(const float2* part_ml, const float* part_acc, const float2* tail_ml,
                                                  const float* tail_acc, float* o, int G, int S2, int St) {
  __shared__ float fs[kMergeMax];
  __shared__ float lsum;
  const int64_t uhg = blockIdx.x;              // (unit, head) * G + q-head
  const int64_t uh = uhg / G;
  const int g = (int)(uhg % G);
  const int d = threadIdx.x;
  if (threadIdx.x < 64) {
    // wave 0: maxima and weights of the S2 + St ranges
    const int s = threadIdx.x;
    float m = -INFINITY, l = 0.0f;
    if (s < S2) {
      const float2 v = part_ml[(uh * S2 + s) * G + g];
      m = v.x; l = v.y;
    }
    float mt = -INFINITY, lt = 0.0f;
    if (s < St) {
      const float2 v = tail_ml[(uh * St + s) * G + g];
      mt = v.x; lt = v.y;
    }
    const float M = wave_max(fmaxf(m, mt));
    const float f = m == -INFINITY ? 0.0f : exp2_fast(m - M);
    const float ft = mt == -INFINITY ? 0.0f : exp2_fast(mt - M);
    if (s < S2) fs[s] = f;
    if (s < St) fs[64 + s] = ft;
    // the sum of f_s l_s in a fixed order (lane order, then the tail)
    const float L = wave_sum(f * l) + wave_sum(ft * lt);
    if (s == 0) lsum = L;
  }
  __syncthreads();
  float acc = 0.0f;
  const float* pa = part_acc + (uh * S2 * G + g) * kHeadDim + d;
#pragma unroll 8
  for (int s = 0; s < S2; ++s) acc = fmaf(fs[s], pa[(int64_t)s * G * kHeadDim], acc);
  if (St > 0) {
    const float* ta = tail_acc + (uh * St * G + g) * kHeadDim + d;
#pragma unroll 8
    for (int s = 0; s < St; ++s) acc = fmaf(fs[64 + s], ta[(int64_t)s * G * kHeadDim], acc);
  }
  o[uhg * kHeadDim + d] = acc / lsum;
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

constexpr size_t kLdsLimit = 158 * 1024;  // dynamic part; the static part is under 2 KB of the 160 KB

// Waves per workgroup: 8 (two tokens per lane) when two workgroups fit a
// compute unit's LDS, else 16 (one token per lane, one workgroup).
static int decode_waves(int G, int A, bool f32, int codec) {
  return 2 * (dec_lds(G, A, f32, 8, codec).total + 2048) <= 160 * 1024 ? 8 : 16;
}

template <int DT, int G, int NW, int CD>
static int launch_stream_nw(const DecArgs& a, unsigned grid, hipStream_t st) {
  static size_t done = 0;
  const size_t lds = dec_lds(G, a.A, DT == ANCHORKV_F32, NW, CD).total;
  if (lds > kLdsLimit) return fail(ANCHORKV_E_SHAPE, "decode: q_per_kv * anchors too large for LDS");
  if (int rc = set_dyn_lds(reinterpret_cast<const void*>(&k_dec_stream<DT, G, NW, CD>), lds, &done)) return rc;
  k_dec_stream<DT, G, NW, CD><<<grid, 64 * NW, lds, st>>>(a);
  AKV_CHECK_LAUNCH("k_dec_stream");
  return 0;
}

template <int DT, int G>
static int launch_stream(const DecArgs& a, unsigned grid, hipStream_t st) {
  const bool nw8 = decode_waves(G, a.A, DT == ANCHORKV_F32, a.codec) == 8;
  if (a.codec == ANCHORKV_CODEC_HADAMARD_LM)
    return nw8 ? launch_stream_nw<DT, G, 8, ANCHORKV_CODEC_HADAMARD_LM>(a, grid, st)
               : launch_stream_nw<DT, G, 16, ANCHORKV_CODEC_HADAMARD_LM>(a, grid, st);
  return nw8 ? launch_stream_nw<DT, G, 8, ANCHORKV_CODEC_AFFINE>(a, grid, st)
             : launch_stream_nw<DT, G, 16, ANCHORKV_CODEC_AFFINE>(a, grid, st);
}

template <int DT>
static int decode_impl(const anchorkv_plan_info& p, const void* cache_v, const void* q, float* o, void* ws_v,
                       hipStream_t st, const void* K_tail = nullptr, const void* V_tail = nullptr, int n_tail = 0,
                       int tail_cap = 0) {
  const uint8_t* cache = reinterpret_cast<const uint8_t*>(cache_v);
  uint8_t* ws = reinterpret_cast<uint8_t*>(ws_v);
  const DecodeWs w = decode_ws_layout(p);
  const int U = p.units, H = p.H, G = p.G, A = p.A, S2 = w.S2;
  if (int rc = decode_supports(p)) return rc;
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
  a.joint = p.joint; a.R_total = p.R_total;
  a.codec = p.params.codec;
  a.signs = make_uint4(p.params.hadamard_signs[0], p.params.hadamard_signs[1], p.params.hadamard_signs[2],
                       p.params.hadamard_signs[3]);
  a.force_part = n_tail > 0 ? 1 : 0;
  a.G = G;
  a.rope = p.params.rope;
  a.rope_theta = p.params.rope_theta;
  const unsigned grid = (unsigned)((int64_t)U * H * S2);
  int rc = 0;
  if (a.rope) {
    // the weight-table kernel while its [G][A] table fits, else the one that
    // rebuilds every value row
    const size_t wl = (size_t)G * A * sizeof(unsigned long long);
    if (wl <= (size_t)kRopeWMaxBytes) {
      static size_t done = 0;
      if (int rc2 = set_dyn_lds(reinterpret_cast<const void*>(&k_dec_rope_w<DT>), wl, &done)) return rc2;
      k_dec_rope_w<DT><<<grid, 256, wl, st>>>(a);
      AKV_CHECK_LAUNCH("k_dec_rope_w");
    } else {
      k_dec_rope<DT><<<grid, 256, 0, st>>>(a);
      AKV_CHECK_LAUNCH("k_dec_rope");
    }
  } else switch (G) {
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
    k_dec_merge<<<(unsigned)((int64_t)U * H * G), kHeadDim, 0, st>>>(a.part_ml, a.part_acc, tml, tacc, o, G, S2, w.St);
    AKV_CHECK_LAUNCH("k_dec_merge");
    prof_mark(st, "dec_tail");
    return 0;
  }
  if (S2 > 1) {
    k_dec_merge<<<(unsigned)((int64_t)U * H * G), kHeadDim, 0, st>>>(a.part_ml, a.part_acc, nullptr, nullptr, o, G, S2, 0);
    AKV_CHECK_LAUNCH("k_dec_merge");
  }
  prof_mark(st, "dec_stream");
  return 0;
}

int decode_blocks_per_cu(int G, int A, bool f32, int codec) {
  // 8-wave workgroups two per compute unit, 16-wave ones alone (four waves per SIMD either way)
  return decode_waves(G, A, f32, codec) == 8 ? 2 : 1;
}

int decode_supports(const anchorkv_plan_info& p) {
  if (p.G > kMaxG) return fail(ANCHORKV_E_SHAPE, "anchorkv_plan: decode supports q_per_kv <= %d", kMaxG);
  const bool f32 = p.dtype == ANCHORKV_F32;
  if (p.params.rope && p.params.codec != ANCHORKV_CODEC_AFFINE)
    return fail(ANCHORKV_E_SHAPE, "anchorkv_plan: pre-RoPE keys need the group-affine codec");
  // the pre-RoPE kernel reads anchors from memory: no anchor limit from LDS
  if (!p.params.rope &&
      dec_lds(p.G, p.A, f32, decode_waves(p.G, p.A, f32, p.params.codec), p.params.codec).total > kLdsLimit)
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

// ---- allocation-free decode.  Its workspace (the per-range partials when a
// head is split into several token ranges) lives in a file-scope device array
// that each GPU holds until the process ends.  Host code must not pass the
// array's name to a kernel (in host code it is a stand-in, not a device
// address): the device address is looked up once per device with
// hipGetSymbolAddress and kept.
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];
constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices] = {};

static int static_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(ANCHORKV_E_HIP, "anchorkv_decode_attn_noalloc: no current device (or device index >= %d)", kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(ANCHORKV_E_HIP, "anchorkv_decode_attn_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return 0;
}

int run_decode_noalloc(const anchorkv_plan_info& p, const void* cache, const void* q, float* o, void* stream) {
  // the decode without a tail uses the workspace up to the tail partials
  const int64_t need = decode_ws_layout(p).tail_ml;
  if (need > (int64_t)kStaticScratchBytes)
    return fail(ANCHORKV_E_SMALL_BUFFER,
                "anchorkv_decode_attn_noalloc: this plan needs %lld bytes of workspace, the static workspace holds %zu",
                (long long)need, kStaticScratchBytes);
  void* ws = nullptr;
  if (int rc = static_scratch(&ws)) return rc;
  return run_decode(p, cache, q, o, ws, stream);
}

int run_decode_tail(const anchorkv_plan_info& p, const void* cache, const void* q, const void* K_tail,
                    const void* V_tail, int n_tail, int tail_cap, float* o, void* ws, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (p.dtype == ANCHORKV_BF16)
    return decode_impl<ANCHORKV_BF16>(p, cache, q, o, ws, st, K_tail, V_tail, n_tail, tail_cap);
  return decode_impl<ANCHORKV_F32>(p, cache, q, o, ws, st, K_tail, V_tail, n_tail, tail_cap);
}

}  // namespace akv
