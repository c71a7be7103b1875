// Nearest-anchor assignment for bf16 inputs (gfx950): cosine similarity of
// every token with every anchor of its head on MFMA, fused argmax, then the
// projection gamma = <x, x_a>/||x_a||^2 and ||x - gamma x_a||^2 (Pith review,
// "What carries the argument": nearest anchor by cosine, least-squares
// coefficient; AnchorKV-adapted page, "Evidence": anchors map to themselves
// with coefficient 1 and zero residual).
//
// Layout of the work: one block of 8 or 16 waves owns a run of token
// tiles (64 tokens per wave) of one (unit, side, head); each wave keeps its 64
// tokens as MFMA A fragments in registers and walks the anchors,
// which sit in LDS for the whole block (<= 512 anchors; larger sets are
// processed in parts, see below).  c[t][a] = <x_t, x_a> comes from
// v_mfma_f32_16x16x32_bf16 on exact bf16 operands and is scaled by
// 1/||x_a|| in f32.
//
// Argmax key: the bits of the scaled cosine with the 5 lowest mantissa bits
// replaced by (31 - anchor block) (at most 32 blocks of 16 anchors per part),
// compared as signed integers, so one v_max_i32 per element keeps both the
// running maximum and (within a lane's column) the lowest anchor block on
// ties.  A key differs from its value by less than 2^-18 relative, so two
// anchors can only swap order when their cosines are closer than 2^-17
// (7.6e-6) relative, which the tie rule of the method (top-2 margin below
// 1e-5 relative) already excuses.  The 16 anchor columns of a token are then
// reduced with a DPP row maximum; the lowest column holding it (a ballot and
// a bit scan) wins equal keys.
//
// Blocks of 8 waves run two per compute unit when the anchors of a part fit
// twice in LDS (up to ~300 anchors), so that one block's loads (its anchors,
// its first token tile) overlap the other's compute; larger parts use 16-wave
// blocks, one per compute unit.
//
// Anchor sets larger than kAssignResMax are processed in parts inside the
// kernel: every token tile walks the parts, keeping each token's best as a
// 64-bit key (monotone cosine bits << 32 | ~index), so the tokens are read
// once.
#pragma once

#include "device_common.hpp"
#include "obs_pipe.hpp"

#include <climits>
#include <type_traits>

namespace akv {

constexpr int kAssignSlot = 2 * 64 * 4;   // per-wave LDS bytes: token scalars of a 64-token tile
// Dynamic LDS of a block with `waves` waves over `nA` anchors.
// (multi: anchors in parts; a 64-bit running best per token of each wave)
inline size_t assign_lds_bytes(int nA, int waves, bool multi = false) {
  const size_t rows = (size_t)((nA + 15) / 16) * 16;
  return rows * kHeadDim * 2 + rows * 8 + (size_t)waves * kAssignSlot + (multi ? (size_t)waves * 64 * 8 : 0);
}

struct AssignArgs {
  const uint16_t* K;
  const uint16_t* V;
  uint8_t* cache;
  int64_t stride, off_anchor_k, off_anchor_v;
  const float2* anorm;       // [U][2][H][A] (||x_a||^2, 1/||x_a|| or 0)
  const int* anchor_of;      // [U][H][N]
  int* aidx;                 // [U][2][H][N]
  float* gam;                // [U][2][H][N] unrounded gamma
  float* rn2;                // [U][2][H][N] ||x - gamma x_a||^2
  float* vn2;                // [U][H][N] ||v||^2
  const float* score;        // [U][H][N]
  float* util;               // [U][2][H][N] (value side written here)
  int H, N, A, a0, a1;       // anchors [a0, a1) of this launch
  int tiles_per_block, nblk;  // token tiles per block, blocks per (unit, side, head)
};

// Projection epilogue of one 16-token row block: lane (col, kg) holds
// coordinates st*32 + kg*8 .. +7 of token row col in xf[st]; `a` is the
// token's anchor index (already forced for anchor tokens), `arow(c)` returns
// 16-byte chunk c of the anchor row (LDS tile or global memory); na2 is
// ||x_a||^2 and score the token's observation score (value side).
// <x, x_a> and ||x||^2 come from v_dot2_f32_bf16 on the bf16 pairs (exact
// products, f32 sums); on the value side ||r||^2 = ||x||^2 - gamma <x, x_a>,
// recomputed coordinate by coordinate when that cancels by more than 10x.
template <typename RowPtr>
__device__ __forceinline__ void assign_project(const AssignArgs& g, int u, int side, int h, int t, int a, bool is_anchor,
                                               float na2, float score, const bf16x8 (&xf)[4], RowPtr arow, int kg) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  const int64_t uh = (int64_t)u * g.H + h;
  uint4 ach[4];
  for (int st = 0; st < 4; ++st) ach[st] = arow(st * 4 + kg);
  float dot = 0.0f, xx = 0.0f;
  for (int st = 0; st < 4; ++st) {
    const uint4 xw = __builtin_bit_cast(uint4, xf[st]);
    const uint32_t xv[4] = {xw.x, xw.y, xw.z, xw.w};
    const uint32_t av[4] = {ach[st].x, ach[st].y, ach[st].z, ach[st].w};
    for (int i = 0; i < 4; ++i) {
      const bf16x2 xp = __builtin_bit_cast(bf16x2, xv[i]);
      dot = __builtin_amdgcn_fdot2_f32_bf16(xp, __builtin_bit_cast(bf16x2, av[i]), dot, false);
      if (side == 1) xx = __builtin_amdgcn_fdot2_f32_bf16(xp, xp, xx, false);
    }
  }
  dot = sum_rows4(dot);
  float gm = na2 > 0.0f ? dot / na2 : 0.0f;
  if (is_anchor) gm = 1.0f;
  float r2 = 0.0f;
  if (side == 1) {
    xx = sum_rows4(xx);
    r2 = fmaxf(fmaf(-gm, dot, xx), 0.0f);
    const bool cancels = !is_anchor && r2 < 0.1f * xx;
    if (__builtin_amdgcn_ballot_w64(cancels) != 0) {
      float d2 = 0.0f;
      for (int st = 0; st < 4; ++st) {
        const uint4 xw = __builtin_bit_cast(uint4, xf[st]);
        const uint32_t xv[4] = {xw.x, xw.y, xw.z, xw.w};
        const uint32_t av[4] = {ach[st].x, ach[st].y, ach[st].z, ach[st].w};
        for (int i = 0; i < 4; ++i) {
          const float r0 = fmaf(-gm, __uint_as_float(av[i] << 16), __uint_as_float(xv[i] << 16));
          const float r1 = fmaf(-gm, __uint_as_float(av[i] & 0xFFFF0000u), __uint_as_float(xv[i] & 0xFFFF0000u));
          d2 = fmaf(r0, r0, fmaf(r1, r1, d2));
        }
      }
      d2 = sum_rows4(d2);
      if (cancels) r2 = d2;
    }
    if (is_anchor) r2 = 0.0f;
  }
  if (kg == 0 && t < g.N) {
    const int64_t i = ((int64_t)u * 2 * g.H + side * g.H + h) * g.N + t;
    g.aidx[i] = a;
    g.gam[i] = gm;
    g.rn2[i] = r2;
    if (side == 1) {
      // value channel of the utility: score_t ||r_V|| (anchors ineligible)
      g.vn2[uh * g.N + t] = xx;
      g.util[i] = is_anchor ? -1.0f : score * sqrtf(r2);
    }
  }
}

// Anchor tile layout: chunk c of row r at r*16 + (c ^ (r & 15)), so the 16
// rows an MFMA B fragment read touches land on 16 distinct chunk positions.
__device__ __forceinline__ int res_phys(int r, int c) { return r * 16 + (c ^ (r & 15)); }

// MULTI: the anchors of the head exceed one LDS part (kAssignResMax); every
// token tile walks all parts (each copied into LDS in turn, the tokens staying
// in registers), keeping each token's best as a 64-bit key (monotone cosine
// bits << 32 | ~anchor index: lowest index on equal keys); the projection
// then reads the winning anchor row from the cache.  The tokens are read from
// memory once, whatever the number of parts.
template <bool MULTI, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void k_assign_res(AssignArgs g) {
  constexpr int kTile = 64 * WAVES;   // tokens per block tile
  using M = Mfma<ANCHORKV_BF16>;
  constexpr int D = kHeadDim;
  extern __shared__ __attribute__((aligned(16))) uint4 dyn_lds[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, kg = lane >> 4;
  int bid = blockIdx.x;
  const int blk = bid % g.nblk; bid /= g.nblk;
  const int h = bid % g.H; bid /= g.H;
  const int side = bid % 2;
  const int u = bid / 2;
  const int N = g.N, A = g.A;
  const int64_t uh = (int64_t)u * g.H + h;
  const int pa = MULTI ? kAssignResMax : A;           // anchors per part
  const int nparts = (A + pa - 1) / pa;
  const int nab_max = (pa + 15) >> 4;
  uint4* As = dyn_lds;                                            // [nab*16 rows][16 chunks], swizzled
  float* inv_s = reinterpret_cast<float*>(As + nab_max * 16 * 16);  // [nab*16] 1/||x_a||
  float* na2_s = inv_s + nab_max * 16;                                // [nab*16] ||x_a||^2
  // per wave: [64] anchor_of of its tokens (then the chosen anchor, bit 31 =
  // anchor token), [64] observation scores
  int* selfs = reinterpret_cast<int*>(na2_s + nab_max * 16) + wave * (kAssignSlot / 4);
  float* scs = reinterpret_cast<float*>(selfs + 64);
  // MULTI: [64] running best key of the wave's tokens
  unsigned long long* runb = reinterpret_cast<unsigned long long*>(
                                 reinterpret_cast<int*>(na2_s + nab_max * 16) + WAVES * (kAssignSlot / 4)) +
                             wave * 64;
  const uint16_t* X = (side ? g.V : g.K) + uh * N * D;
  const uint16_t* AX = reinterpret_cast<const uint16_t*>(g.cache + (int64_t)u * g.stride +
                                                         (side ? g.off_anchor_v : g.off_anchor_k)) +
                       (int64_t)h * A * D;
  const float2* an = g.anorm + ((int64_t)u * 2 * g.H + side * g.H + h) * A;

  const int ntiles_hs = (N + kTile - 1) / kTile;
  const int tile0 = blk * g.tiles_per_block;
  const int tile1 = min(ntiles_hs, tile0 + g.tiles_per_block);

  auto load_tokens = [&](int tile, bf16x8 (&xf)[4][4]) {
    const int tb = tile * kTile + wave * 64;
    for (int rb = 0; rb < 4; ++rb) {
      const int t = min(tb + rb * 16 + col, N - 1);
      for (int st = 0; st < 4; ++st) xf[rb][st] = M::load(X + (int64_t)t * D + st * 32 + kg * 8);
    }
  };
  // anchors [a0, a1) into LDS (rows beyond a1 repeat the last one: padding
  // rows copy the last anchor's row and 1/||x_a||, tie with it and lose on
  // the column, so they never win)
  auto load_part = [&](int a0, int a1) {
    const int nA = a1 - a0, nab = (nA + 15) >> 4;
    for (int jj = wave; jj < nab * 4; jj += WAVES) {
      const int r = jj * 4 + (lane >> 4);               // tile row of this lane's chunk
      const int c = (lane & 15) ^ (r & 15);             // its logical chunk
      dma16(AX + (int64_t)(a0 + min(r, nA - 1)) * D + c * 8, As + jj * 64);
    }
    for (int i = threadIdx.x; i < nab * 16; i += blockDim.x) {
      const float2 v = an[a0 + min(i, nA - 1)];
      inv_s[i] = v.y;
      na2_s[i] = v.x;
    }
  };

  bf16x8 xf[4][4];
  if (!MULTI) load_part(0, A);
  if (tile0 < tile1) load_tokens(tile0, xf);
  if (!MULTI) {
    __builtin_amdgcn_s_waitcnt(AKV_VMCNT_IMM(0));
    __syncthreads();
  }

  // Running maximum of the keys as signed integers: for non-negative
  // cosines the float bits order like the values, so v_max_i32 needs no NaN
  // canonicalisation.  A wave holding a token whose best key over the part's
  // anchors is negative (every cosine <= 0, rare) redoes the search with
  // sign-corrected keys; the test is on the token's row maximum, since a
  // lane's own column sees only A/16 anchors and is often all negative.
  // the mask lives in a VGPR so that (bits & mask) | tag is one v_and_or_b32
  // (an empty asm makes the value opaque; the move itself is the compiler's,
  // so its hazard checks see every instruction)
  unsigned keymask = 0xffffffe0u;
  __asm__ volatile("" : "+v"(keymask));
  auto search = [&](const bf16x8 (&xt)[4][4], int (&best)[4][4], int nab, auto mono_tag) {
    constexpr bool mono = decltype(mono_tag)::value;
    for (int rb = 0; rb < 4; ++rb)
      for (int r = 0; r < 4; ++r) best[rb][r] = INT_MIN;
    auto mfmas = [&](int ab, f32x4 (&acc)[4]) {
      for (int rb = 0; rb < 4; ++rb) acc[rb] = f32x4{0, 0, 0, 0};
      for (int st = 0; st < 4; ++st) {
        const bf16x8 bf = bits_to_frag(As[res_phys(ab * 16 + col, st * 4 + kg)]);
        for (int rb = 0; rb < 4; ++rb) acc[rb] = M::mma(xt[rb][st], bf, acc[rb]);
      }
    };
    auto keys = [&](int ab, const f32x4 (&acc)[4]) {
      const float inv = inv_s[ab * 16 + col];
      const unsigned tag = 31u - (unsigned)ab;
      for (int rb = 0; rb < 4; ++rb)
        for (int r = 0; r < 4; ++r) {
          unsigned b = __float_as_uint(acc[rb][r] * inv);
          if constexpr (mono) b ^= (unsigned)((int)b >> 31) & 0x7FFFFFFFu;
          const int key = (int)((b & keymask) | tag);
          best[rb][r] = max(best[rb][r], key);
        }
    };
    f32x4 acc0[4];
    for (int ab = 0; ab < nab; ++ab) { mfmas(ab, acc0); keys(ab, acc0); }
  };

  for (int tile = tile0; tile < tile1; ++tile) {
    // per-token scalars of the epilogue, copied into this wave's LDS slots
    // while the search runs (no registers held across it)
    {
      const int t = min(tile * kTile + wave * 64 + lane, N - 1);
      dma4(g.anchor_of + uh * N + t, selfs);
      if (side) dma4(g.score + uh * N + t, scs);
    }
    // MULTI: running best of each token (written by the lane that takes it)
    if (MULTI) runb[lane] = 0ull;
    for (int part = 0; part < nparts; ++part) {
      const int a0 = part * pa, a1 = min(A, a0 + pa);
      const int nab = (a1 - a0 + 15) >> 4;
      if (MULTI) {
        __syncthreads();          // every wave is done with the previous part
        load_part(a0, a1);
        __builtin_amdgcn_s_waitcnt(AKV_VMCNT_IMM(0));
        __syncthreads();
      }
      int best[4][4];
      int mk[4][4];   // row (token) maxima of the keys
      auto row_maxima = [&]() {
        for (int rb = 0; rb < 4; ++rb)
          for (int r = 0; r < 4; ++r) mk[rb][r] = row_max_i32(best[rb][r]);
      };
      search(xf, best, nab, std::false_type{});
      row_maxima();
      bool neg = false;
      for (int rb = 0; rb < 4; ++rb)
        for (int r = 0; r < 4; ++r) neg |= mk[rb][r] < 0;
      if (__builtin_amdgcn_ballot_w64(neg) != 0) {
        search(xf, best, nab, std::true_type{});
        row_maxima();
      }
      __builtin_amdgcn_s_waitcnt(AKV_VMCNT_IMM(0));   // this wave's copies of selfs / scs
      // ---- reduce the 16 anchor columns of every token: row maximum of the
      // keys, lowest column holding it; lanes col < 4 of row kg take token
      // rb*16 + kg*4 + col
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        int wv[4];
        for (int r = 0; r < 4; ++r) {
          const int m = mk[rb][r];
          const unsigned long long eq = __builtin_amdgcn_ballot_w64(best[rb][r] == m);
          const unsigned bits = (unsigned)(eq >> (kg * 16)) & 0xFFFFu;   // never 0: the row holds its maximum
          wv[r] = a0 + __builtin_ctz(bits) + 16 * (31 - (m & 31));
        }
        if (col < 4) {
          if constexpr (MULTI) {
            // (one static index per pass: a select over mk would become a
            // private-memory array lookup)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              if (col == r) {
                // signed-monotone key -> unsigned order, then ~index for lowest-index ties
                const unsigned long long key64 =
                    ((unsigned long long)(((unsigned)mk[rb][r] & keymask) ^ 0x80000000u) << 32) |
                    (unsigned long long)(0xFFFFFFFFu - (unsigned)wv[r]);
                const int tl = rb * 16 + kg * 4 + r;
                runb[tl] = max(runb[tl], key64);
              }
            }
          } else {
            const int w = col == 0 ? wv[0] : col == 1 ? wv[1] : col == 2 ? wv[2] : wv[3];
            const int tl = rb * 16 + kg * 4 + col;   // token of the wave's tile
            const int self = selfs[tl];
            selfs[tl] = self >= 0 ? (int)(0x80000000u | (unsigned)self) : w;
          }
        }
      }
    }
    if constexpr (MULTI) {
      // each token's entry was written by its own lane: one lane per token now
      __builtin_amdgcn_s_waitcnt(0xC07F);
      __builtin_amdgcn_wave_barrier();
      const int w = (int)(0xFFFFFFFFu - (unsigned)(runb[lane] & 0xFFFFFFFFull));
      const int self = selfs[lane];
      selfs[lane] = self >= 0 ? (int)(0x80000000u | (unsigned)self) : w;
    }
    // ---- projection of every token onto its anchor
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's selfs writes done
    __builtin_amdgcn_wave_barrier();
    for (int rb = 0; rb < 4; ++rb) {
      const int t = tile * kTile + wave * 64 + rb * 16 + col;
      const int sa = selfs[rb * 16 + col];
      const bool is_anchor = sa < 0;
      const int a = sa & 0x7FFFFFFF;
      if constexpr (MULTI)
        assign_project(g, u, side, h, t, a, is_anchor, an[a].x, scs[rb * 16 + col], xf[rb],
                       [&](int c) { return *reinterpret_cast<const uint4*>(AX + (int64_t)a * D + c * 8); }, kg);
      else
        assign_project(g, u, side, h, t, a, is_anchor, na2_s[a], scs[rb * 16 + col], xf[rb],
                       [&](int c) { return As[res_phys(a, c)]; }, kg);
    }
    // this wave's LDS slots are rewritten by the next tile's copies
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_wave_barrier();
    if (tile + 1 < tile1) load_tokens(tile + 1, xf);
  }
}

}  // namespace akv
