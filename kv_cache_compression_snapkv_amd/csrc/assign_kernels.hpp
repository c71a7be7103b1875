// Nearest-anchor assignment for bf16 inputs (gfx950): cosine similarity of
// every token with every anchor of its head on MFMA, fused argmax, then the
// projection gamma = <x, x_a>/||x_a||^2 and ||x - gamma x_a||^2 (Pith review,
// "What carries the argument": nearest anchor by cosine, least-squares
// coefficient; AnchorKV-adapted page, "Evidence": anchors map to themselves
// with coefficient 1 and zero residual).
//
// Layout of the work: one block of 8 waves owns a run of 512-token tiles of
// one (unit, side, head); each wave keeps its 64 tokens as MFMA A fragments in
// registers (the next tile's prefetched alongside) and walks the anchors,
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
// reduced through a small per-wave LDS array, lowest column first on equal
// keys.
//
// Anchor sets larger than kAssignResMax are processed in parts: each part
// folds its per-token winner into a 64-bit key (monotone cosine bits << 32 |
// ~index) with a global atomicMax (order independent, so deterministic), and
// k_assign_proj then does the projection for every token.
#pragma once

#include "device_common.hpp"
#include "obs_pipe.hpp"

#include <climits>

namespace akv {

constexpr int kAssignTile = 512;     // tokens per block tile (8 waves x 64)

struct AssignArgs {
  const uint16_t* K;
  const uint16_t* V;
  uint8_t* cache;
  int64_t stride, off_anchor_k, off_anchor_v, off_words;
  const float2* anorm;       // [U][2][H][A] (||x_a||^2, 1/||x_a|| or 0)
  const int* anchor_of;      // [U][H][N]
  int* aidx;                 // [U][2][H][N]
  float* gam;                // [U][2][H][N] unrounded gamma
  float* rn2;                // [U][2][H][N] ||x - gamma x_a||^2
  float* vn2;                // [U][H][N] ||v||^2
  const float* score;        // [U][H][N]
  float* util;               // [U][2][H][N] (value side written here)
  unsigned long long* best64;  // [U][2][H][N] packed winners of the parts
  int H, N, A, a0, a1;       // anchors [a0, a1) of this launch
  int tiles_per_block, nblk;  // token tiles per block, blocks per (unit, side, head)
};

// Projection epilogue of one 16-token row block: lane (col, kg) holds
// coordinates st*32 + kg*8 .. +7 of token row col in xf[st]; `a` is the
// token's anchor index (already forced for anchor tokens), `ar` points to the
// anchor row (LDS tile or global memory).
template <typename RowPtr>
__device__ __forceinline__ void assign_project(const AssignArgs& g, int u, int side, int h, int t, int a, bool is_anchor,
                                               const bf16x8 (&xf)[4], RowPtr arow, int kg) {
  const int64_t uh = (int64_t)u * g.H + h;
  float dot = 0.0f, xx = 0.0f;
  float xs[32], as_[32];
  for (int st = 0; st < 4; ++st) {
    const uint4 av = arow(st * 4 + kg);
    uint16_t ab[8];
    __builtin_memcpy(ab, &av, 16);
    for (int e = 0; e < 8; ++e) {
      xs[st * 8 + e] = (float)xf[st][e];
      as_[st * 8 + e] = bf2f(ab[e]);
      dot = fmaf(xs[st * 8 + e], as_[st * 8 + e], dot);
      xx = fmaf(xs[st * 8 + e], xs[st * 8 + e], xx);
    }
  }
  dot += __shfl_xor(dot, 16, 64);
  dot += __shfl_xor(dot, 32, 64);
  const float na2 = g.anorm[((int64_t)u * 2 * g.H + side * g.H + h) * g.A + a].x;
  float gm = na2 > 0.0f ? dot / na2 : 0.0f;
  if (is_anchor) gm = 1.0f;
  float r2 = 0.0f;
  for (int i = 0; i < 32; ++i) {
    const float rr = fmaf(-gm, as_[i], xs[i]);
    r2 = fmaf(rr, rr, r2);
  }
  r2 += __shfl_xor(r2, 16, 64);
  r2 += __shfl_xor(r2, 32, 64);
  if (is_anchor) r2 = 0.0f;
  if (side == 1) {
    xx += __shfl_xor(xx, 16, 64);
    xx += __shfl_xor(xx, 32, 64);
  }
  if (kg == 0 && t < g.N) {
    const int64_t i = ((int64_t)u * 2 * g.H + side * g.H + h) * g.N + t;
    g.aidx[i] = a;
    g.gam[i] = gm;
    g.rn2[i] = r2;
    uint32_t* words = reinterpret_cast<uint32_t*>(g.cache + (int64_t)u * g.stride + g.off_words);
    words[((int64_t)h * g.N + t) * 2 + side] = (uint32_t)a | ((uint32_t)f2h_sat(gm) << 16);
    if (side == 1) {
      // value channel of the utility: score_t ||r_V|| (anchors ineligible)
      g.vn2[uh * g.N + t] = xx;
      g.util[i] = is_anchor ? -1.0f : g.score[uh * g.N + t] * sqrtf(r2);
    }
  }
}

template <bool PARTIAL>
__global__ __launch_bounds__(512) void k_assign_res(AssignArgs g) {
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
  const int N = g.N;
  const int64_t uh = (int64_t)u * g.H + h;
  const int nA = g.a1 - g.a0;
  const int nab = (nA + 15) >> 4;
  uint4* As = dyn_lds;                                        // [nab*16 rows][16 chunks], swizzled
  float* inv_s = reinterpret_cast<float*>(As + nab * 16 * 16);  // [nab*16]
  int* red = reinterpret_cast<int*>(inv_s + nab * 16) + wave * (16 * 17);  // per wave [16 tokens][17]
  const uint16_t* X = (side ? g.V : g.K) + uh * N * D;
  const uint16_t* AX = reinterpret_cast<const uint16_t*>(g.cache + (int64_t)u * g.stride +
                                                         (side ? g.off_anchor_v : g.off_anchor_k)) +
                       (int64_t)h * g.A * D;
  const float2* an = g.anorm + ((int64_t)u * 2 * g.H + side * g.H + h) * g.A;

  // ---- anchors of this part into LDS (rows beyond nA repeat the last one)
  {
    const DmaLane dl(lane);
    for (int jj = wave; jj < nab * 4; jj += 8) {
      const int r = min(jj * 4 + dl.rsub, nA - 1);
      dma16(AX + (int64_t)(g.a0 + r) * D + ((jj & 1) ? dl.c1 : dl.c0) * 8, As + jj * 64);
    }
    // padding rows copy the last anchor (row and 1/||x_a||): they tie with it
    // and lose on the column, so they never win
    for (int i = threadIdx.x; i < nab * 16; i += blockDim.x) inv_s[i] = an[g.a0 + min(i, nA - 1)].y;
    __builtin_amdgcn_s_waitcnt(AKV_VMCNT_IMM(0));
    __syncthreads();
  }

  const int ntiles_hs = (N + kAssignTile - 1) / kAssignTile;
  const int tile0 = blk * g.tiles_per_block;
  const int tile1 = min(ntiles_hs, tile0 + g.tiles_per_block);

  auto load_tokens = [&](int tile, bf16x8 (&xf)[4][4]) {
    const int tb = tile * kAssignTile + wave * 64;
    for (int rb = 0; rb < 4; ++rb) {
      const int t = min(tb + rb * 16 + col, N - 1);
      for (int st = 0; st < 4; ++st) xf[rb][st] = M::load(X + (int64_t)t * D + st * 32 + kg * 8);
    }
  };

  // Running maximum of the keys as signed integers: for non-negative
  // cosines the float bits order like the values, so v_max_i32 needs no NaN
  // canonicalisation.  A wave holding a token whose best key is negative
  // (every cosine <= 0, rare) redoes the search with sign-corrected keys.
  // the mask lives in a VGPR so that (bits & mask) | tag is one v_and_or_b32
  unsigned keymask;
  __asm__("v_mov_b32 %0, 0xffffffe0" : "=v"(keymask));
  auto search = [&](const bf16x8 (&xt)[4][4], int (&best)[4][4], bool mono) {
    for (int rb = 0; rb < 4; ++rb)
      for (int r = 0; r < 4; ++r) best[rb][r] = INT_MIN;
    for (int ab = 0; ab < nab; ++ab) {
      bf16x8 bf[4];
      for (int st = 0; st < 4; ++st) bf[st] = bits_to_frag(As[obs_phys(ab * 16 + col, st * 4 + kg)]);
      const float inv = inv_s[ab * 16 + col];
      const unsigned tag = 31u - (unsigned)ab;
      for (int rb = 0; rb < 4; ++rb) {
        f32x4 acc = {0, 0, 0, 0};
        for (int st = 0; st < 4; ++st) acc = M::mma(xt[rb][st], bf[st], acc);
        for (int r = 0; r < 4; ++r) {
          unsigned b = __float_as_uint(acc[r] * inv);
          if (mono) b ^= (unsigned)((int)b >> 31) & 0x7FFFFFFFu;
          const int key = (int)((b & keymask) | tag);
          best[rb][r] = max(best[rb][r], key);
        }
      }
    }
  };

  bf16x8 xf[4][4], xn[4][4];
  if (tile0 < tile1) load_tokens(tile0, xf);
  for (int tile = tile0; tile < tile1; ++tile) {
    if (tile + 1 < tile1) load_tokens(tile + 1, xn);
    int best[4][4];
    search(xf, best, false);
    bool neg = false;
    for (int rb = 0; rb < 4; ++rb)
      for (int r = 0; r < 4; ++r) neg |= best[rb][r] < 0;
    const bool mono = __builtin_amdgcn_ballot_w64(neg) != 0;
    if (mono) search(xf, best, true);
    // ---- per 16-token row block: reduce the 16 anchor columns, then project
    for (int rb = 0; rb < 4; ++rb) {
      for (int r = 0; r < 4; ++r) red[(kg * 4 + r) * 17 + col] = best[rb][r];
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes done
      __builtin_amdgcn_wave_barrier();
      int win = 0, wkey = INT_MIN;
      if (lane < 16) {
        for (int c = 0; c < 16; ++c) {
          const int k = red[lane * 17 + c];
          if (k > wkey) { wkey = k; win = c; }   // strict: lowest column on equal keys
        }
        win = g.a0 + win + 16 * (31 - (wkey & 31));
      }
      const int tt = tile * kAssignTile + wave * 64 + rb * 16;
      if constexpr (PARTIAL) {
        if (lane < 16 && tt + lane < N) {
          // signed-monotone key -> unsigned order, then ~index for lowest-index ties
          const unsigned long long key64 = ((unsigned long long)(((unsigned)wkey & keymask) ^ 0x80000000u) << 32) |
                                           (unsigned long long)(0xFFFFFFFFu - (unsigned)win);
          atomicMax(g.best64 + ((int64_t)u * 2 * g.H + side * g.H + h) * N + tt + lane, key64);
        }
      } else {
        int a = __shfl(win, col, 64);
        const int t = tt + col;
        const int self = g.anchor_of[uh * N + min(t, N - 1)];
        const bool is_anchor = self >= 0;
        if (is_anchor) a = self;
        assign_project(g, u, side, h, t, a, is_anchor, xf[rb],
                       [&](int c) { return As[obs_phys(a - g.a0, c)]; }, kg);
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // reads of red done before the next row block writes it
      __builtin_amdgcn_wave_barrier();
    }
    if (tile + 1 < tile1)
      for (int rb = 0; rb < 4; ++rb)
        for (int st = 0; st < 4; ++st) xf[rb][st] = xn[rb][st];
  }
}

// Projection after a partitioned anchor search: one 4-lane group per token
// (64 tokens per 256-thread block; lanes (col, kg) as in the MFMA layout).
__global__ __launch_bounds__(256) void k_assign_proj(AssignArgs g, int64_t total) {
  constexpr int D = kHeadDim;
  const int lane = threadIdx.x & 63;
  const int kg = lane >> 4;
  const int64_t tok = (int64_t)blockIdx.x * 64 + (threadIdx.x >> 6) * 16 + (lane & 15);  // over [U][2][H][N]
  const bool live = tok < total;
  const int64_t tk = live ? tok : total - 1;
  const int t = (int)(tk % g.N);
  int64_t rest = tk / g.N;
  const int h = (int)(rest % g.H); rest /= g.H;
  const int side = (int)(rest % 2);
  const int u = (int)(rest / 2);
  const int64_t uh = (int64_t)u * g.H + h;
  const uint16_t* X = (side ? g.V : g.K) + (uh * g.N + t) * D;
  const uint16_t* AX = reinterpret_cast<const uint16_t*>(g.cache + (int64_t)u * g.stride +
                                                         (side ? g.off_anchor_v : g.off_anchor_k)) +
                       (int64_t)h * g.A * D;
  bf16x8 xf[4];
  for (int st = 0; st < 4; ++st) xf[st] = Mfma<ANCHORKV_BF16>::load(X + st * 32 + kg * 8);
  const int self = g.anchor_of[uh * g.N + t];
  const bool is_anchor = self >= 0;
  const unsigned long long key = g.best64[tk];
  const int a = is_anchor ? self : (int)(0xFFFFFFFFu - (unsigned)(key & 0xFFFFFFFFull));
  assign_project(g, u, side, h, live ? t : g.N, a, is_anchor, xf,
                 [&](int c) { return *reinterpret_cast<const uint4*>(AX + (int64_t)a * D + c * 8); }, kg);
}

}  // namespace akv
