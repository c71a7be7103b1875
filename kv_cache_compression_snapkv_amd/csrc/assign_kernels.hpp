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
// Argmax key: the scaled cosine with its 5 lowest mantissa bits replaced by
// a tag, the anchor's position among the 32 anchors a lane sees in an epoch
// of 8 blocks (31 - position, so that among equal positive keys the earlier
// anchor wins), compared as floats (v_max3_f32 orders negative values
// correctly; the tag only decides between keys equal after masking).  A key
// differs from its value by less than 2^-18 relative, so two anchors can only
// swap order when their cosines are closer than 2^-17 (7.6e-6) relative,
// which the tie rule of the method (top-2 margin below 1e-5 relative) already
// excuses.  Each epoch's winner is compared with the token's best so far, and
// the four lanes that share a token merge their bests at the end (larger
// key, then lower index).
//
// Blocks of 8 waves run two per compute unit when the anchors of a part fit
// twice in LDS (up to ~300 anchors), so that one block's loads (its anchors,
// its first token tile) overlap the other's compute; larger parts use 16-wave
// blocks, one per compute unit.
//
// Anchor sets larger than kAssignResMax are processed inside the kernel in
// the fewest equal parts of at most kAssignPartMax anchors: every token tile
// walks the parts with each token's best carried in registers from part to
// part, so the tokens are read once, and odd tiles walk them backwards so
// that the part left in LDS by one tile starts the next.
#pragma once

#include "device_common.hpp"
#include "obs_pipe.hpp"

#include <climits>
#include <type_traits>

namespace akv {

constexpr int kAssignSlot = 2 * 64 * 4;   // per-wave LDS bytes: token scalars of a 64-token tile
// Dynamic LDS of a block with `waves` waves over `nA` anchors (one part).
inline size_t assign_lds_bytes(int nA, int waves) {
  const size_t rows = (size_t)((nA + 15) / 16) * 16;
  return rows * kHeadDim * 2 + rows * 8 + (size_t)waves * kAssignSlot;
}

// max(a, b, c) of finite floats in one instruction (fmaxf on values made from
// integer bits would first be canonicalised, one more instruction per input)
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float d;
  __asm__("v_max3_f32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}
// (v, a) <- the better of the two candidates (larger value, then lower index);
// the candidates are this lane's and its partner's, in either order.
__device__ __forceinline__ void take_better(float& v, int& a, float v0, int a0, float v1, int a1) {
  const bool first = v0 > v1 || (v0 == v1 && a0 < a1);
  v = first ? v0 : v1;
  a = first ? a0 : a1;
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
  int xcd_groups;             // > 0: XCD-grouped order (see k_assign_res), the number of (unit, side, head) groups
  int part;                   // MULTI: anchors per LDS part (a multiple of 16)
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
// token tile walks all parts (each copied into LDS in turn, the tokens and
// their running bests staying in registers); the projection then reads the
// winning anchor row from the cache.  The tokens are read from memory once,
// whatever the number of parts.
template <bool MULTI, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void k_assign_res(AssignArgs g) {
  constexpr int kTile = 64 * WAVES;   // tokens per block tile
  using M = Mfma<ANCHORKV_BF16>;
  constexpr int D = kHeadDim;
  extern __shared__ __attribute__((aligned(16))) uint4 dyn_lds[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, kg = lane >> 4;
  // Workgroups go to the eight XCDs in turn (workgroup b to XCD b mod 8).
  // With xcd_groups > 0 the blocks of one (unit, side, head) all go to one
  // XCD and run there together, so the anchor parts they reload tile after
  // tile stay in that XCD's L2: XCD x takes groups x, x + 8, ... one after
  // the other, nblk blocks each (nblk is one per compute unit of an XCD).
  int bid = blockIdx.x;
  if (g.xcd_groups > 0) {
    const int x = bid & 7, k = bid >> 3;
    const int grp = x + 8 * (k / g.nblk);
    if (grp >= g.xcd_groups) return;   // padding of the last round (whole block)
    bid = grp * g.nblk + k % g.nblk;
  }
  const int blk = bid % g.nblk; bid /= g.nblk;
  const int h = bid % g.H; bid /= g.H;
  const int side = bid % 2;
  const int u = bid / 2;
  const int N = g.N, A = g.A;
  const int64_t uh = (int64_t)u * g.H + h;
  const int pa = MULTI ? g.part : A;                  // anchors per part
  const int nparts = (A + pa - 1) / pa;
  const int nab_max = (pa + 15) >> 4;
  uint4* As = dyn_lds;                                            // [nab*16 rows][16 chunks], swizzled
  float* inv_s = reinterpret_cast<float*>(As + nab_max * 16 * 16);  // [nab*16] 1/||x_a||
  float* na2_s = inv_s + nab_max * 16;                                // [nab*16] ||x_a||^2
  // per wave: [64] anchor_of of its tokens (>= 0: an anchor token), [64]
  // observation scores
  int* selfs = reinterpret_cast<int*>(na2_s + nab_max * 16) + wave * (kAssignSlot / 4);
  float* scs = reinterpret_cast<float*>(selfs + 64);
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
  // rows copy the last anchor's row and 1/||x_a|| and so tie with it)
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

  // (bits & keymask) | tag is one v_and_or_b32 with the mask in a VGPR (an
  // empty asm makes the value opaque; the move itself is the compiler's, so
  // its hazard checks see every instruction)
  unsigned keymask = 0xffffffe0u;
  __asm__ volatile("" : "+v"(keymask));

  // Anchors of one part: blocks of 16 anchors in epochs of 8 blocks.  The
  // MFMA takes the anchors as its A operand and the tokens as B, so lane
  // (col, kg) receives anchors ab*16 + kg*4 + r (r = 0..3) of token
  // rb*16 + col: its four keys of a block all belong to one token and fold
  // into that token's running key with two v_max3_f32.  At the end of an
  // epoch the running key (masked value, tag = epoch position) is compared
  // with the token's best so far (bv, bix) and restarted.
  // A block's 1/||x_a|| are read before its MFMAs, and the next block's first
  // A fragment before its keys are formed, so both LDS reads are in flight
  // while the block's MFMA and VALU work runs.
  auto search_part = [&](int nab, int gab0, float (&bv)[4], int (&bix)[4]) {
    bf16x8 af0 = bits_to_frag(As[res_phys(col, kg)]);
    for (int e = 0; e < nab; e += 8) {
      float run[4];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j > 0 && e + j >= nab) break;
        const int ab = e + j;
        const float4 inv = *reinterpret_cast<const float4*>(inv_s + ab * 16 + kg * 4);
        f32x4 acc[4];
        for (int rb = 0; rb < 4; ++rb) acc[rb] = f32x4{0, 0, 0, 0};
        for (int st = 0; st < 4; ++st) {
          const bf16x8 af = st == 0 ? af0 : bits_to_frag(As[res_phys(ab * 16 + col, st * 4 + kg)]);
          for (int rb = 0; rb < 4; ++rb) acc[rb] = M::mma(af, xf[rb][st], acc[rb]);
        }
        // rows past the part's padded blocks are never read: the last block
        // reads its own first fragment again
        af0 = bits_to_frag(As[res_phys(min(ab + 1, nab - 1) * 16 + col, kg)]);
        const float iv[4] = {inv.x, inv.y, inv.z, inv.w};
        for (int rb = 0; rb < 4; ++rb) {
          float k[4];
          for (int r = 0; r < 4; ++r)
            k[r] = __uint_as_float((__float_as_uint(acc[rb][r] * iv[r]) & keymask) | (31u - (unsigned)(j * 4 + r)));
          if (j == 0)
            run[rb] = max3f(max3f(k[0], k[1], k[2]), k[3], k[3]);
          else
            run[rb] = max3f(max3f(run[rb], k[0], k[1]), k[2], k[3]);
        }
      }
      const int ge = gab0 + e;          // first block of this epoch (parts need not start on an epoch of the head)
      for (int rb = 0; rb < 4; ++rb) {
        const unsigned b = __float_as_uint(run[rb]);
        const float m = __uint_as_float(b & keymask);
        // the larger value, the earlier epoch on equal values (epochs come
        // in increasing order in one part; parts are visited in either order)
        if (m > bv[rb] || (MULTI && m == bv[rb] && ge < (bix[rb] >> 5))) {
          bv[rb] = m;
          bix[rb] = (ge << 5) | (int)(b & 31u);
        }
      }
    }
  };

  int loaded = -1;   // the part in LDS (MULTI)
  for (int tile = tile0; tile < tile1; ++tile) {
    // per-token scalars of the epilogue, copied into this wave's LDS slots
    // while the search runs (no registers held across it)
    {
      const int t = min(tile * kTile + wave * 64 + lane, N - 1);
      dma4(g.anchor_of + uh * N + t, selfs);
      if (side) dma4(g.score + uh * N + t, scs);
    }
    float bv[4];
    int bix[4];
    for (int rb = 0; rb < 4; ++rb) { bv[rb] = -__builtin_inff(); bix[rb] = 0x7FFFFFFF; }
    // odd tiles walk the parts backwards, so the part in LDS at the end of a
    // tile serves the start of the next one without a reload
    const bool back = MULTI && ((tile - tile0) & 1);
    for (int pi = 0; pi < nparts; ++pi) {
      const int part = back ? nparts - 1 - pi : pi;
      const int a0 = part * pa, a1 = min(A, a0 + pa);
      if (MULTI && part != loaded) {
        __syncthreads();          // every wave is done with the previous part
        load_part(a0, a1);
        __builtin_amdgcn_s_waitcnt(AKV_VMCNT_IMM(0));
        __syncthreads();
        loaded = part;
      }
      search_part((a1 - a0 + 15) >> 4, a0 >> 4, bv, bix);
    }
    // ---- each token's anchor: decode the lane's best (epoch, position),
    // then the larger key over the four lanes of the token (kg = 0..3), the
    // lower index on equal keys.  Rows past the last anchor repeat it; a tie
    // with one of them can only decode past A - 1 and is clamped back.
    int best_a[4];
    for (int rb = 0; rb < 4; ++rb) {
      const int li = 31 - (bix[rb] & 31);
      int a = ((bix[rb] >> 5) + (li >> 2)) * 16 + kg * 4 + (li & 3);
      a = min(a, A - 1);
      float v = bv[rb];
      const auto v32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
      const auto a32 = __builtin_amdgcn_permlane32_swap((unsigned)a, (unsigned)a, false, false);
      take_better(v, a, __uint_as_float(v32[0]), (int)a32[0], __uint_as_float(v32[1]), (int)a32[1]);
      const auto v16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
      const auto a16 = __builtin_amdgcn_permlane16_swap((unsigned)a, (unsigned)a, false, false);
      take_better(v, a, __uint_as_float(v16[0]), (int)a16[0], __uint_as_float(v16[1]), (int)a16[1]);
      best_a[rb] = a;
    }
    __builtin_amdgcn_s_waitcnt(AKV_VMCNT_IMM(0));   // this wave's copies of selfs / scs
    // ---- projection of every token onto its anchor (anchor tokens onto themselves)
    for (int rb = 0; rb < 4; ++rb) {
      const int t = tile * kTile + wave * 64 + rb * 16 + col;
      const int self = selfs[rb * 16 + col];
      const bool is_anchor = self >= 0;
      const int a = is_anchor ? self : best_a[rb];
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
