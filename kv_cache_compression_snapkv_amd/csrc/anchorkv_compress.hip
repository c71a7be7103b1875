// End-of-prefill compression pass (gfx950).
//
// Launch sequence per call (all units at once, one stream, no host sync):
//   headers -> obs STATS -> ml combine -> obs SCORE -> o combine ->
//   anchor selection (+ anchor copy, norms) -> nearest-anchor assignment per
//   side (MFMA similarity, fused argmax and projection) -> obs UTIL ->
//   top-R radix select (3 digit passes) -> counts -> chunk scan -> flags +
//   record order -> quantise + pack.
// Sources: Pith review of AnchorKV ("What carries the argument",
// "Assumptions & free parameters"); AnchorKV-adapted page ("Evidence",
// "Adaptation notes").
#include "launch_common.hpp"
#include "obs_kernels.hpp"
#include "obs_pipe.hpp"
#include "assign_kernels.hpp"

namespace akv {


// Fill kernel (used instead of a memset so the sequence stays capture-safe).
__global__ void k_zero_u32(unsigned* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// Zeroes nseg segments of len words, seg_stride words apart.
__global__ void k_zero_seg(unsigned* p, int64_t len, int64_t seg_stride, int64_t nseg) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < len * nseg) p[(i / len) * seg_stride + i % len] = 0u;
}

// ------------------------------------------------------------------ headers
__global__ void k_headers(UnitHeader hd, uint8_t* cache, int64_t stride) {
  const int u = blockIdx.x;
  const int i = threadIdx.x;  // 64 threads x 4 bytes
  uint32_t v;
  if (i == (int)(offsetof(UnitHeader, unit_index) / 4)) v = (uint32_t)u;
  else v = reinterpret_cast<const uint32_t*>(&hd)[i];
  reinterpret_cast<uint32_t*>(cache + (int64_t)u * stride)[i] = v;
}

// ------------------------------------------------------------ stats combines
// m (log2 domain) and l over key splits -> (m, 1/l); deterministic order.
__global__ void k_ml_combine(const float2* part, float2* ml, int S1, int GQp, int GQ, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int q = (int)(i % GQp);
  const int64_t uh = i / GQp;
  if (q >= GQ) { ml[i] = make_float2(0.0f, 0.0f); return; }
  float m = -INFINITY;
  for (int s = 0; s < S1; ++s) m = fmaxf(m, part[(uh * S1 + s) * GQp + q].x);
  float l = 0.0f;
  for (int s = 0; s < S1; ++s) {
    float2 v = part[(uh * S1 + s) * GQp + q];
    if (v.x > -INFINITY) l += v.y * exp2_fast(v.x - m);
  }
  ml[i] = make_float2(m, 1.0f / l);
}

// o = sum of split partials (fixed order), its bf16 hi/lo split and ||o||^2.
// One 128-thread block per (unit, head, query).
__global__ void k_o_combine(const float* part, float* o, uint16_t* ohl, float* oo, int S1, int GQp) {
  const int64_t row = blockIdx.x;   // (uh, q)
  const int q = (int)(row % GQp);
  const int64_t uh = row / GQp;
  const int d = threadIdx.x;
  // the partials are added in split order; with several splits their loads
  // are issued 8 at a time
  const float* pp = part + (uh * S1 * GQp + q) * kHeadDim + d;
  const int64_t ps = (int64_t)GQp * kHeadDim;
  float v = pp[0];
  for (int s0 = 1; s0 < S1; s0 += 8) {
    float x[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = s0 + k < S1 ? pp[(s0 + k) * ps] : 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (s0 + k < S1) v += x[k];
  }
  o[row * kHeadDim + d] = v;
  const uint16_t hi = f2bf(v);
  const uint16_t lo = f2bf(v - bf2f(hi));
  ohl[((uh * 2 + 0) * GQp + q) * kHeadDim + d] = hi;
  ohl[((uh * 2 + 1) * GQp + q) * kHeadDim + d] = lo;
  __shared__ float red[2];
  float sq = wave_sum(v * v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = sq;
  __syncthreads();
  if (threadIdx.x == 0) oo[row] = red[0] + red[1];
}

// -------------------------------------------------------------- block scans
// Exclusive scan of one int per thread over a 1024-thread block; returns the
// exclusive prefix and writes the total to *total.
__device__ int block_excl_scan(int v, int* sh /*[32]*/, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int x = v;
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int w = 0; w < nw; ++w) { int t = sh[w]; sh[w] = acc; acc += t; }
    sh[31] = acc;
  }
  __syncthreads();
  const int r = sh[wave] + x - v;
  *total = sh[31];
  __syncthreads();
  return r;
}

// Adds 1 to hist[bin] for every active lane.  Lanes of a wave that share a
// bin add their count with one atomic (the common case in the top digits of
// nearby values, where one bin would otherwise take 64 serialised LDS
// atomics); after four such rounds the remaining lanes add one by one.
__device__ __forceinline__ void hist_add_wave(unsigned* hist, unsigned bin, bool act) {
  const int lane = threadIdx.x & 63;
  unsigned long long pend = __ballot(act);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (pend == 0) return;
    const int lead = __builtin_ctzll(pend);
    const unsigned lb = (unsigned)__builtin_amdgcn_readlane((int)bin, lead);
    const unsigned long long same = __ballot(act && bin == lb);
    if (lane == lead) atomicAdd(&hist[lb], (unsigned)__popcll(same));
    act = act && bin != lb;
    pend &= ~same;
  }
  if (act) atomicAdd(&hist[bin], 1u);
}

__device__ __forceinline__ int lanes_before(unsigned long long m) {
  return (int)__builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
}

// Radix-select step over a histogram in LDS: finds the bucket b (scanning from
// the top) where the running count first reaches `need`; returns b and the
// count strictly above it.  Block-parallel: each thread owns a run of
// consecutive buckets (highest first), one exclusive scan finds the run.
__device__ void find_bucket(const unsigned* hist, int nbins, unsigned need, int* sh, int* out_b, unsigned* out_above) {
  const int nt = blockDim.x;
  const int per = (nbins + nt - 1) / nt;
  const int hi = nbins - 1 - threadIdx.x * per;  // this thread's buckets: hi, hi-1, ..., hi-per+1
  unsigned local = 0;
  for (int k = 0; k < per; ++k) {
    const int b = hi - k;
    if (b >= 0) local += hist[b];
  }
  int tot;
  const unsigned above0 = (unsigned)block_excl_scan((int)local, sh, &tot);
  if (above0 < need && above0 + local >= need) {
    unsigned cum = above0;
    for (int k = 0; k < per; ++k) {
      const int b = hi - k;
      if (b < 0) break;
      if (cum + hist[b] >= need) { *out_b = b; *out_above = cum; break; }
      cum += hist[b];
    }
  }
  __syncthreads();
}

// The k positions t < L with the largest keys key(t) (ties to the lower
// position), ascending into out[0..k): a 3-pass radix select over the 32-bit
// keys (11 + 11 + 10 bits), then an ordered compaction in which each wave
// walks one contiguous range of positions 64 at a time, ranks from ballots.
// Whole block; key(t) is read once per pass and twice in the compaction.
template <typename KeyF>
__device__ void select_top(int L, int k, KeyF key, int* out, unsigned* hist, int* sh, int* s_b, unsigned* s_above) {
  const int tid = threadIdx.x, nt = blockDim.x;
  unsigned prefix = 0, need = (unsigned)k;
  if (k > 0) {
    const int shifts[3] = {21, 10, 0};
    const int widths[3] = {11, 11, 10};
    for (int p = 0; p < 3; ++p) {
      for (int b = tid; b < kHistBins; b += nt) hist[b] = 0;
      __syncthreads();
      const unsigned hmask = p == 0 ? 0u : (0xFFFFFFFFu << (shifts[p] + widths[p]));
      for (int t0 = 0; t0 < L; t0 += nt) {  // wave-uniform trip count
        const int t = t0 + tid;
        const unsigned kv = t < L ? key(t) : 0u;
        hist_add_wave(hist, (kv >> shifts[p]) & ((1u << widths[p]) - 1), t < L && (kv & hmask) == (prefix & hmask));
      }
      __syncthreads();
      if (tid == 0) { *s_b = 0; *s_above = 0; }
      __syncthreads();
      find_bucket(hist, 1 << widths[p], need, sh, s_b, s_above);
      prefix = prefix | ((unsigned)*s_b << shifts[p]);
      need = need - *s_above;
      __syncthreads();
    }
  }
  const unsigned T_key = prefix;
  const int lane = tid & 63, wave = tid >> 6, nw = nt >> 6;
  const int seg = (((L + nw - 1) / nw) + 63) & ~63;
  const int s0 = min(L, wave * seg), s1 = min(L, s0 + seg);
  int ng = 0, nti = 0;  // wave totals (uniform)
  if (k > 0)
    for (int t0 = s0; t0 < s1; t0 += 64) {
      const int t = t0 + lane;
      const unsigned kv = t < s1 ? key(t) : 0u;
      ng += __popcll(__ballot(t < s1 && kv > T_key));
      nti += __popcll(__ballot(t < s1 && kv == T_key));
    }
  int tot;
  const int tie_pre = __builtin_amdgcn_readlane(block_excl_scan(lane == 0 ? nti : 0, sh, &tot), 0);
  // selected in this range: all greater + ties while tie rank < need
  const int take_ties = k > 0 ? max(0, min(nti, (int)need - tie_pre)) : 0;
  const int sel_pre = __builtin_amdgcn_readlane(block_excl_scan(lane == 0 && k > 0 ? ng + take_ties : 0, sh, &tot), 0);
  if (k > 0) {
    int o = sel_pre, tr = tie_pre;
    for (int t0 = s0; t0 < s1; t0 += 64) {
      const int t = t0 + lane;
      const unsigned kv = t < s1 ? key(t) : 0u;
      const bool tie = t < s1 && kv == T_key;
      const unsigned long long tm = __ballot(tie);
      const bool sel = (t < s1 && kv > T_key) || (tie && tr + lanes_before(tm) < (int)need);
      const unsigned long long sm = __ballot(sel);
      if (sel) out[o + lanes_before(sm)] = t;
      o += __popcll(sm);
      tr += __popcll(tm);
    }
  }
}

// ---------------------------------------------------------- anchor selection
constexpr int kSelectLdsMaxL = 32768;   // pooled score in LDS up to this many positions (128 KB)
// One 1024-thread block per (unit, head).  score -> pooled (window sum of
// odd width `pool`, 7 by default, over non-window positions) -> top k_s (radix select on the f32 bits,
// ties to the lower position) -> k_u stratified picks over the remaining
// positions (pick i = remaining[floor((2i+1) M / (2 k_u))]) -> + window ->
// positions ascending, anchor_of map, anchor copies, norms.  With LP the
// pooled score stays in LDS (dynamic, L floats), else it goes through the
// workspace.
template <int DT, bool LP>
__global__ __launch_bounds__(1024) void k_select(const void* Kv, const void* Vv, const float* score, float* pooled,
                                                 uint8_t* cache, int64_t stride, int64_t off_ak, int64_t off_av,
                                                 int64_t off_pos, int* anchor_of, float2* anorm, int H, int N, int W,
                                                 int k_s, int k_u, int A, int pool, int mode, int* clist) {
  using T = typename Elem<DT>::T;
  constexpr int D = kHeadDim;
  __shared__ unsigned hist[kHistBins];
  __shared__ int sh[32];
  __shared__ int s_b;
  __shared__ unsigned s_above;
  __shared__ int s_pos[4096];  // scored + uniform positions (A <= 4096 is checked on the host)
  __shared__ float stg[1024 + kMaxPool - 1];
  extern __shared__ float plds[];
  const int h = blockIdx.x % H;
  const int u = blockIdx.x / H;
  const int64_t uh = (int64_t)u * H + h;
  const int L = N - W;
  const float* sc = score + uh * N;
  float* pl = LP ? plds : pooled + uh * N;
  const int tid = threadIdx.x, nt = blockDim.x;

  // coverage anchors (mode 1, 2; see k_cover): the picks list of this head
  int* cl = clist + uh * (int64_t)(k_s + k_u);
  if (mode != 2) {
  // pooled_t = score_{t-hw} + ... + score_{t+hw} over [0, L), hw = pool/2
  // (zeros outside, added in position order)
  const int hw = pool >> 1;
  if constexpr (LP) {
    // whole score in LDS (all loads in flight at once), pooled values in
    // registers, then written over it
    static_assert(kSelectLdsMaxL % 1024 == 0, "per-thread slots");
    constexpr int PER = kSelectLdsMaxL / 1024;
    for (int t = tid; t < L; t += nt) pl[t] = sc[t];
    __syncthreads();
    float pv[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int t = tid + k * nt;
      float v = 0.0f;
      if (t < L)
        for (int j = 0; j < pool; ++j) {
          const int x = t - hw + j;
          v += (x >= 0 && x < L) ? pl[x] : 0.0f;
        }
      pv[k] = v;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < PER; ++k)
      if (tid + k * nt < L) pl[tid + k * nt] = pv[k];
    __syncthreads();
  } else {
    // 1024-position chunks of the score staged with an hw-position halo
    for (int t0 = 0; t0 < L; t0 += nt) {
      for (int i = tid; i < nt + 2 * hw; i += nt) {
        const int x = t0 - hw + i;
        stg[i] = (x >= 0 && x < L) ? sc[x] : 0.0f;
      }
      __syncthreads();
      const int t = t0 + tid;
      if (t < L) {
        float v = 0.0f;
        for (int k = 0; k < pool; ++k) v += stg[tid + k];
        pl[t] = v;
      }
      __syncthreads();
    }
  }

  // the k_s largest pooled scores (f32 bits of non-negative values), ties to
  // the lower position, ascending into s_pos
  select_top(L, k_s, [&](int t) { return __float_as_uint(pl[t]); }, s_pos, hist, sh, &s_b, &s_above);
  __syncthreads();
  if (mode == 1) {   // scored positions only: the coverage picks follow (k_cover)
    for (int i = tid; i < k_s; i += nt) cl[i] = s_pos[i];
    return;
  }
  // uniform picks: the c-th remaining position is c + j, j = first index with scored[j] - j > c
  const int M = L - k_s;
  for (int i = tid; i < k_u; i += nt) {
    const int64_t c = ((2ll * i + 1) * M) / (2ll * k_u);
    int lo = 0, hi = k_s;  // first j in [0, k_s] with (j == k_s) or scored[j] - j > c
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if ((int64_t)s_pos[mid] - mid > c) hi = mid; else lo = mid + 1;
    }
    s_pos[k_s + i] = (int)(c + lo);
  }
  } else {
    // mode 2: the scored positions (ascending) and the coverage picks (in
    // round order, distinct) from the list; the picks go to s_pos[k_s..]
    // ascending (rank = picks below)
    for (int i = tid; i < k_s; i += nt) s_pos[i] = cl[i];
    for (int i = tid; i < k_u; i += nt) {
      const int v = cl[k_s + i];
      int rank = 0;
      for (int j = 0; j < k_u; ++j) rank += cl[k_s + j] < v ? 1 : 0;
      s_pos[k_s + rank] = v;
    }
  }
  const int lane = tid & 63, wave = tid >> 6, nw = nt >> 6;
  __syncthreads();
  // merge scored (sorted) and uniform (sorted) into anchor order (ranks by
  // binary search, then written over s_pos once every read is done), then the
  // window
  int* pos_out = reinterpret_cast<int*>(cache + (int64_t)u * stride + off_pos) + (int64_t)h * A;
  {
    int mv[4], mr[4];  // k_s + k_u < 4096 = 4 per thread
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = tid + k * nt;
      mv[k] = -1;
      mr[k] = 0;
      if (i < k_s + k_u) {
        const int v = s_pos[i];
        int rank;
        if (i < k_s) {  // count uniform picks below v
          int lo = 0, hi = k_u;
          while (lo < hi) { int mid = (lo + hi) >> 1; if (s_pos[k_s + mid] < v) lo = mid + 1; else hi = mid; }
          rank = i + lo;
        } else {
          int lo = 0, hi = k_s;
          while (lo < hi) { int mid = (lo + hi) >> 1; if (s_pos[mid] < v) lo = mid + 1; else hi = mid; }
          rank = (i - k_s) + lo;
        }
        mv[k] = v;
        mr[k] = rank;
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (mv[k] >= 0) s_pos[mr[k]] = mv[k];
    for (int i = tid; i < W; i += nt) s_pos[k_s + k_u + i] = L + i;
  }
  int* ao = anchor_of + uh * N;
  for (int t = tid; t < N; t += nt) ao[t] = -1;
  __syncthreads();  // s_pos in anchor order; ao cleared (block-visible)
  __threadfence_block();
  for (int i = tid; i < A; i += nt) {
    pos_out[i] = s_pos[i];
    ao[s_pos[i]] = i;
  }
  // copy anchor rows and their norms: 16-byte chunks, 64/CPR rows per wave
  // instruction, the row's lanes summed by a DPP row reduction
  constexpr int CPR = D * (int)sizeof(T) / 16;   // chunks per row: 16 (bf16) or 32 (f32)
  constexpr int RPW = 64 / CPR;
  constexpr int EPC = 16 / (int)sizeof(T);       // elements per chunk
  const int rsub = lane / CPR, ch = lane % CPR;
  const T* Kp = reinterpret_cast<const T*>(Kv) + uh * N * D;
  const T* Vp = reinterpret_cast<const T*>(Vv) + uh * N * D;
  T* AK = reinterpret_cast<T*>(cache + (int64_t)u * stride + off_ak) + (int64_t)h * A * D;
  T* AV = reinterpret_cast<T*>(cache + (int64_t)u * stride + off_av) + (int64_t)h * A * D;
  for (int i0 = wave * RPW; i0 < A; i0 += nw * RPW) {
    const int i = i0 + rsub;
    float sk = 0.0f, sv = 0.0f;
    if (i < A) {
      const int t = s_pos[i];
      const uint4 xk = *reinterpret_cast<const uint4*>(Kp + (int64_t)t * D + ch * EPC);
      const uint4 xv = *reinterpret_cast<const uint4*>(Vp + (int64_t)t * D + ch * EPC);
      *reinterpret_cast<uint4*>(AK + (int64_t)i * D + ch * EPC) = xk;
      *reinterpret_cast<uint4*>(AV + (int64_t)i * D + ch * EPC) = xv;
      T ek[EPC], ev[EPC];
      __builtin_memcpy(ek, &xk, 16);
      __builtin_memcpy(ev, &xv, 16);
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        const float fk = Elem<DT>::f(ek[e]), fv = Elem<DT>::f(ev[e]);
        sk = fmaf(fk, fk, sk);
        sv = fmaf(fv, fv, sv);
      }
    }
    sk = row_sum(sk);
    sv = row_sum(sv);
    if constexpr (CPR == 32) {  // rows of 32 lanes: add the other half-row
      sk += __shfl_xor(sk, 16, 64);
      sv += __shfl_xor(sv, 16, 64);
    }
    if (i < A && ch == 0) {
      anorm[((int64_t)u * 2 * H + h) * A + i] = make_float2(sk, sk > 0.0f ? 1.0f / sqrtf(sk) : 0.0f);
      anorm[((int64_t)u * 2 * H + H + h) * A + i] = make_float2(sv, sv > 0.0f ? 1.0f / sqrtf(sv) : 0.0f);
    }
  }
}

// ------------------------------------------------- coverage anchor picks
// anchor_mode == ANCHORKV_ANCHORS_COVER (Pith review, "Reading between the
// lines": anchors placed for coverage, by k-means or furthest-point picks, in
// place of the uniform ones), read as furthest-point sampling on the keys in
// batched rounds.  One 1024-thread block per (unit, head), between k_select's
// first pass (scored positions into the list) and its second (final order,
// anchor map, copies):
//  * mc[t], t < L: largest signed cosine of key t to the scored and window
//    anchors, on MFMA (anchor rows from the keys as the A operand, 16 tokens
//    per row block as B), then +inf at the scored anchors;
//  * each round: the b positions with the lowest mc, ties to the lower one
//    (select_top on the complemented order-preserving bits), are appended to
//    the list and get mc = +inf; mc then takes the maximum with their cosines
//    (every round but the last).
constexpr int kCoverMaxA = 4096;   // A <= 4096 is checked on the host

__device__ __forceinline__ float frag_sq(float v) { return v * v; }
__device__ __forceinline__ float frag_sq(bf16x8 v) {
  float s = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float f = (float)v[e];
    s = fmaf(f, f, s);
  }
  return s;
}
// maximum over the four 16-lane rows (every lane gets it)
__device__ __forceinline__ float max_rows4(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

template <int DT>
__global__ __launch_bounds__(1024) void k_cover(const void* Kv, int* clist, float* mcb, int H, int N, int W, int k_s,
                                                int k_u, int rounds) {
  using T = typename Elem<DT>::T;
  using MS = Mfma<DT>;
  constexpr int D = kHeadDim;
  constexpr int NST = D / MS::KSTEP;
  constexpr int RB = DT == ANCHORKV_BF16 ? 2 : 1;   // 16-token row blocks per wave
  constexpr int TW = 16 * RB;                       // tokens per wave
  __shared__ unsigned hist[kHistBins];
  __shared__ int sh[32];
  __shared__ int s_b;
  __shared__ unsigned s_above;
  __shared__ int s_new[kCoverMaxA];     // the round's picks, ascending
  __shared__ float s_inv[kCoverMaxA];   // 1/||x_a|| of the anchors being added (0 for a zero row)
  const int h = blockIdx.x % H, u = blockIdx.x / H;
  const int64_t uh = (int64_t)u * H + h;
  const int L = N - W;
  const int tid = threadIdx.x, nt = blockDim.x;
  const int lane = tid & 63, wave = tid >> 6, nw = nt >> 6;
  const int col = lane & 15, kg = lane >> 4;
  const T* X = reinterpret_cast<const T*>(Kv) + uh * (int64_t)N * D;
  int* cl = clist + uh * (int64_t)(k_s + k_u);
  float* mc = mcb + uh * (int64_t)N;

  // mc[t] <- cosine to the na anchors at positions apos(i) (first), else the
  // larger of mc[t] and that
  auto update = [&](auto apos, int na, bool first) {
    for (int i = tid; i < na; i += nt) {
      const T* r = X + (int64_t)apos(i) * D;
      float s2 = 0.0f;
      for (int d = 0; d < D; ++d) {
        const float v = Elem<DT>::f(r[d]);
        s2 = fmaf(v, v, s2);
      }
      s_inv[i] = s2 > 0.0f ? 1.0f / sqrtf(s2) : 0.0f;
    }
    __syncthreads();
    const int nab = (na + 15) >> 4;
    for (int t0 = wave * TW; t0 < L; t0 += nw * TW) {   // wave-uniform
      typename MS::frag xf[RB][NST];
      float xx[RB], run[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int t = min(t0 + rb * 16 + col, L - 1);
        xx[rb] = 0.0f;
        run[rb] = -INFINITY;
#pragma unroll
        for (int st = 0; st < NST; ++st) {
          xf[rb][st] = MS::load(X + (int64_t)t * D + st * MS::KSTEP + kg * MS::KW);
          xx[rb] += frag_sq(xf[rb][st]);
        }
      }
      for (int ab = 0; ab < nab; ++ab) {
        // A operand: anchor row ab*16 + col (rows past the last anchor repeat it)
        const T* arow = X + (int64_t)apos(min(ab * 16 + col, na - 1)) * D;
        f32x4 acc[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) acc[rb] = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int st = 0; st < NST; ++st) {
          const typename MS::frag af = MS::load(arow + st * MS::KSTEP + kg * MS::KW);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) acc[rb] = MS::mma(af, xf[rb][st], acc[rb]);
        }
        // lane (col, kg) holds anchors ab*16 + kg*4 + r of token rb*16 + col
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float iv = s_inv[min(ab * 16 + kg * 4 + r, na - 1)];
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) run[rb] = fmaxf(run[rb], acc[rb][r] * iv);
        }
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const float x2 = sum_rows4(xx[rb]);
        const float m = max_rows4(run[rb]);
        const float c = x2 > 0.0f ? m / sqrtf(x2) : 0.0f;
        const int t = t0 + rb * 16 + col;
        if (kg == 0 && t < L) mc[t] = first ? c : fmaxf(mc[t], c);
      }
    }
    __syncthreads();
  };

  // scored positions (ascending, from k_select's first pass), then the window
  update([&](int i) { return i < k_s ? cl[i] : L + (i - k_s); }, k_s + W, true);
  for (int i = tid; i < k_s; i += nt) mc[cl[i]] = INFINITY;
  __syncthreads();
  const int R = max(1, min(rounds, k_u));
  int done = 0;
  for (int r = 0; r < R && k_u > 0; ++r) {
    const int b = (int)(((int64_t)k_u * (r + 1)) / R - ((int64_t)k_u * r) / R);
    // the b lowest mc first: complement of the order-preserving bits
    select_top(L, b, [&](int t) {
      const unsigned x = __float_as_uint(mc[t]);
      return ~((int)x < 0 ? ~x : (x | 0x80000000u));
    }, s_new, hist, sh, &s_b, &s_above);
    __syncthreads();
    for (int i = tid; i < b; i += nt) {
      cl[k_s + done + i] = s_new[i];
      mc[s_new[i]] = INFINITY;
    }
    done += b;
    __syncthreads();
    if (r + 1 < R) update([&](int i) { return s_new[i]; }, b, false);
  }
}

// ------------------------------------------------- nearest-anchor assignment
// One 256-thread block per (unit, side, head, 256-token tile); each wave owns
// 64 tokens (4 MFMA row blocks) held in registers.  Anchors are staged through
// LDS in chunks; the MFMA tile c[t][a] = <x_t, x_a> is scaled by 1/||x_a|| in
// f32 and a per-lane running argmax keeps the lowest anchor index on ties.
// Then gamma = <x_t, x_a>/||x_a||^2 and ||x_t - gamma x_a||^2 in f32, anchor
// tokens forced onto themselves (gamma 1, residual 0); the pointer word
// (index | fp16 gamma << 16) is written to the cache.
template <int DT> struct AssignCfg {
  static constexpr int AC = DT == ANCHORKV_BF16 ? 256 : 128;   // anchors per LDS chunk
  static constexpr int PAD = DT == ANCHORKV_BF16 ? 8 : 4;
  static constexpr int LDA = kHeadDim + PAD;
};

template <int DT>
__global__ __launch_bounds__(256) void k_assign(const void* Kv, const void* Vv, uint8_t* cache, int64_t stride,
                                               int64_t off_ak, int64_t off_av,
                                               const float2* anorm, const int* anchor_of, int* aidx, float* gam,
                                               float* rn2, float* vn2, const float* score, float* util, int H, int N,
                                               int A, int ntiles) {
  using T = typename Elem<DT>::T;
  using M = Mfma<DT>;
  using frag = typename M::frag;
  using Cfg = AssignCfg<DT>;
  constexpr int D = kHeadDim, NSTEP = D / M::KSTEP, AC = Cfg::AC, LDA = Cfg::LDA;
  __shared__ __attribute__((aligned(16))) T As[AC * LDA];
  __shared__ float inv_s[AC];

  int bid = blockIdx.x;
  const int tile = bid % ntiles; bid /= ntiles;
  const int h = bid % H; bid /= H;
  const int side = bid % 2;
  const int u = bid / 2;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, kg = lane >> 4;
  const int64_t uh = (int64_t)u * H + h;
  const T* X = reinterpret_cast<const T*>(side ? Vv : Kv) + uh * N * D;
  const T* AX = reinterpret_cast<const T*>(cache + (int64_t)u * stride + (side ? off_av : off_ak)) + (int64_t)h * A * D;
  const float2* an = anorm + ((int64_t)u * 2 * H + side * H + h) * A;
  const int tbase = tile * 256 + wave * 64;

  frag xf[4][NSTEP];
  for (int rb = 0; rb < 4; ++rb) {
    const int t = tbase + rb * 16 + col;
    for (int st = 0; st < NSTEP; ++st) {
      const int kk = st * M::KSTEP + kg * M::KW;
      xf[rb][st] = t < N ? M::load(X + (int64_t)t * D + kk) : M::zero();
    }
  }
  float best[4][4];
  int bidx[4][4];
  for (int rb = 0; rb < 4; ++rb)
    for (int r = 0; r < 4; ++r) { best[rb][r] = -INFINITY; bidx[rb][r] = 0; }

  constexpr int EPC = 16 / sizeof(T), CPR = D / EPC;
  for (int c0 = 0; c0 < A; c0 += AC) {
    const int na = min(AC, A - c0);
    for (int ch = threadIdx.x; ch < AC * CPR; ch += blockDim.x) {
      const int r = ch / CPR, cc = ch % CPR;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (r < na) v = *reinterpret_cast<const uint4*>(AX + (int64_t)(c0 + r) * D + cc * EPC);
      *reinterpret_cast<uint4*>(&As[r * LDA + cc * EPC]) = v;
    }
    for (int i = threadIdx.x; i < AC; i += blockDim.x) inv_s[i] = i < na ? an[c0 + i].y : __int_as_float(0x7fc00000);
    __syncthreads();
    const int nab = (na + 15) / 16;
    for (int ab = 0; ab < nab; ++ab) {
      frag bf[NSTEP];
      for (int st = 0; st < NSTEP; ++st) bf[st] = M::load(&As[(ab * 16 + col) * LDA + st * M::KSTEP + kg * M::KW]);
      const float inv = inv_s[ab * 16 + col];  // NaN for padding anchors: never wins
      const int aglob = c0 + ab * 16 + col;
      for (int rb = 0; rb < 4; ++rb) {
        f32x4 acc = {0, 0, 0, 0};
        for (int st = 0; st < NSTEP; ++st) acc = M::mma(xf[rb][st], bf[st], acc);
        for (int r = 0; r < 4; ++r) {
          const float v = acc[r] * inv;
          if (v > best[rb][r]) { best[rb][r] = v; bidx[rb][r] = aglob; }
        }
      }
    }
    __syncthreads();
  }
  // argmax across the 16 anchor-column lanes; lowest index on ties
  for (int rb = 0; rb < 4; ++rb)
    for (int r = 0; r < 4; ++r) {
      float b = best[rb][r];
      int bi = bidx[rb][r];
      for (int o = 1; o < 16; o <<= 1) {
        const float b2 = __shfl_xor(b, o, 64);
        const int i2 = __shfl_xor(bi, o, 64);
        if (b2 > b || (b2 == b && i2 < bi)) { b = b2; bi = i2; }
      }
      bidx[rb][r] = bi;
    }
  // projection epilogue: lane (row col, k-slice kg) holds 32 coordinates of token row col
  for (int rb = 0; rb < 4; ++rb) {
    const int t = tbase + rb * 16 + col;
    // argmax of output row `col` lives in lanes (col/4)*16.., register r = col%4
    int cand[4];
    for (int r = 0; r < 4; ++r) cand[r] = __shfl(bidx[rb][r], (col >> 2) * 16, 64);
    int a = cand[col & 3];
    const int tt = t < N ? t : N - 1;
    const int self = anchor_of[uh * N + tt];
    const bool is_anchor = self >= 0;
    if (is_anchor) a = self;
    float xs[NSTEP * M::KW], as_[NSTEP * M::KW];
    float dot = 0.0f;
    for (int st = 0; st < NSTEP; ++st) {
      const int kk = st * M::KSTEP + kg * M::KW;
      if constexpr (DT == ANCHORKV_BF16) {
        const uint4 av = *reinterpret_cast<const uint4*>(AX + (int64_t)a * D + kk);
        uint16_t ab[8];
        __builtin_memcpy(ab, &av, 16);
        for (int e = 0; e < 8; ++e) {
          xs[st * 8 + e] = (float)xf[rb][st][e];
          as_[st * 8 + e] = bf2f(ab[e]);
        }
      } else {
        xs[st] = xf[rb][st];
        as_[st] = Elem<DT>::f(AX[(int64_t)a * D + kk]);
      }
      for (int e = 0; e < M::KW; ++e) dot = fmaf(xs[st * M::KW + e], as_[st * M::KW + e], dot);
    }
    dot += __shfl_xor(dot, 16, 64);
    dot += __shfl_xor(dot, 32, 64);
    const float na2 = an[a].x;
    float g = na2 > 0.0f ? dot / na2 : 0.0f;
    if (is_anchor) g = 1.0f;
    float r2 = 0.0f;
    for (int i = 0; i < NSTEP * M::KW; ++i) {
      const float rr = fmaf(-g, as_[i], xs[i]);
      r2 = fmaf(rr, rr, r2);
    }
    r2 += __shfl_xor(r2, 16, 64);
    r2 += __shfl_xor(r2, 32, 64);
    if (is_anchor) r2 = 0.0f;
    float xx = 0.0f;
    if (side == 1) {
      for (int i = 0; i < NSTEP * M::KW; ++i) xx = fmaf(xs[i], xs[i], xx);
      xx += __shfl_xor(xx, 16, 64);
      xx += __shfl_xor(xx, 32, 64);
    }
    if (kg == 0 && t < N) {
      const int64_t i = ((int64_t)u * 2 * H + side * H + h) * N + t;
      aidx[i] = a;
      gam[i] = g;
      rn2[i] = r2;
      if (side == 1) {
        // value channel of the utility: score_t ||r_V|| (anchors ineligible)
        vn2[uh * N + t] = xx;
        util[i] = is_anchor ? -1.0f : score[uh * N + t] * sqrtf(r2);
      }
    }
  }
}

// ------------------------------------------------------------- top-R select
// Per (unit, side): choose the R largest utilities over (head, token), ties to
// the lower head then position.  Keys: f32 bits + 1 for eligible (u >= 0),
// 0 for anchors.
//  k_topr_threshold, one 1024-thread block per (unit, side): three radix
//    passes (11/11/10 bits) find the R-th key T and how many keys equal to T
//    are taken; then the counts of keys > T and == T of every group of 1024
//    positions (flat head*N + t order) and their exclusive scans give each
//    group's record base and tie base;
//  k_topr_flag, one wave per group: selects tokens in position order (ballot
//    prefix counts), writes every token's pointer word (anchor index, residual
//    flag, fp16 gamma: plain stores, no read-modify-write), each record's
//    position to the record list and, at every 1024-token chunk start of a
//    head, the number of records before it (the chunk's residual offset).
__device__ __forceinline__ unsigned util_key(float v) { return v >= 0.0f ? __float_as_uint(v) + 1u : 0u; }

constexpr int kToprThreads = 1024;
constexpr int kToprBatch = 16;   // loads in flight per thread (streaming form)
constexpr int kToprKPT = 64;     // keys per thread of the register-resident form
constexpr int kToprCopies = 8;   // histogram copies
constexpr int kToprGroup = 1024; // positions per flag group

// KPT > 0: the block's keys (H*N <= 16 * 64 * KPT) are loaded once into
// registers, wave w holding positions [w*64*KPT, (w+1)*64*KPT) as
// w*64*KPT + 64 s + lane; KPT == 0: every pass streams the utilities.  Wave
// runs are whole groups.
template <int KPT>
__global__ __launch_bounds__(kToprThreads) void k_topr_threshold(const float* util, unsigned* groups, int H, int N,
                                                                 int R) {
  constexpr int NW = kToprThreads / 64;
  constexpr bool REG = KPT > 0;
  constexpr int B = REG ? KPT : kToprBatch;   // keys per batch of a thread
  static_assert((64 * B) % kToprGroup == 0 || kToprGroup % (64 * B) == 0, "batches and groups nest");
  // kToprCopies interleaved histogram copies (bin b of copy c at b*copies + c):
  // keys of one pass share their leading bits, and lanes adding to one LDS
  // address in the same instruction serialise
  __shared__ unsigned lhc[kHistBins * kToprCopies];
  __shared__ unsigned lh[kHistBins];
  __shared__ int sh[32];
  __shared__ int s_b;
  __shared__ unsigned s_above;
  const int us = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t M = (int64_t)H * N;
  const int64_t ngroups = (M + kToprGroup - 1) / kToprGroup;
  const float* up = util + (int64_t)us * M;
  unsigned* gb = groups + (int64_t)us * ngroups * 2;
  unsigned* tn = groups + (int64_t)gridDim.x * ngroups * 2 + (int64_t)us * 2;   // (T, need)
  if (R == 0) {
    if (threadIdx.x == 0) { tn[0] = 0xFFFFFFFFu; tn[1] = 0u; }
    for (int64_t i = threadIdx.x; i < ngroups; i += kToprThreads) { gb[2 * i] = 0u; gb[2 * i + 1] = 0u; }
    return;
  }
  // wave-contiguous runs of positions, whole groups
  const int64_t seg = REG ? (int64_t)64 * KPT : ((M + NW - 1) / NW + kToprGroup - 1) / kToprGroup * kToprGroup;
  const int64_t w0 = (int64_t)wave * seg, w1 = min(M, w0 + seg);
  unsigned keyr[REG ? KPT : 1];
  if constexpr (REG) {
#pragma unroll
    for (int k = 0; k < KPT; ++k) {
      const int64_t i = w0 + 64 * k + lane;
      keyr[k] = i < w1 ? util_key(up[i]) : 0u;
    }
  }
  // keys of the batch starting at j0 (streaming: loaded now, B in flight)
  auto batch = [&](int64_t j0, unsigned (&key)[B]) {
    if constexpr (REG) {
#pragma unroll
      for (int k = 0; k < B; ++k) key[k] = keyr[k];
    } else {
      float v[B];
#pragma unroll
      for (int k = 0; k < B; ++k) {
        const int64_t i = j0 + 64 * k + lane;
        v[k] = i < w1 ? up[i] : -1.0f;
      }
#pragma unroll
      for (int k = 0; k < B; ++k) key[k] = util_key(v[k]);
    }
  };
  // ---- the R-th largest key T and the number of keys equal to T to take
  unsigned prefix = 0u, need = (unsigned)R;
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int width = pass == 2 ? 10 : 11;
    const unsigned hmask = pass == 0 ? 0u : (0xFFFFFFFFu << (shift + width));
    for (int b = threadIdx.x; b < kHistBins * kToprCopies; b += kToprThreads) lhc[b] = 0;
    if (threadIdx.x == 0) { s_b = 0; s_above = 0; }
    __syncthreads();
    const int copy = lane & (kToprCopies - 1);
    for (int64_t j0 = w0; j0 < w1; j0 += 64 * B) {
      unsigned key[B];
      batch(j0, key);
#pragma unroll
      for (int k = 0; k < B; ++k)
        if (key[k] != 0u && (key[k] & hmask) == (prefix & hmask))
          atomicAdd(&lhc[((key[k] >> shift) & ((1u << width) - 1)) * kToprCopies + copy], 1u);
    }
    __syncthreads();
    for (int b = threadIdx.x; b < kHistBins; b += kToprThreads) {
      unsigned sum = 0;
#pragma unroll
      for (int c = 0; c < kToprCopies; ++c) sum += lhc[b * kToprCopies + c];
      lh[b] = sum;
    }
    __syncthreads();
    find_bucket(lh, 1 << width, need, sh, &s_b, &s_above);   // ends with a barrier
    prefix |= (unsigned)s_b << shift;
    need -= s_above;
    __syncthreads();
  }
  const unsigned T = prefix;
  if (threadIdx.x == 0) { tn[0] = T; tn[1] = need; }
  // ---- counts of keys > T and == T per group (kept in LDS), in wave runs
  unsigned* gcnt = lhc;   // [ngroups][2] while ngroups <= 4 * kHistBins; else the group array itself
  const bool in_lds = ngroups * 2 <= (int64_t)kHistBins * kToprCopies;
  unsigned* cnt = in_lds ? gcnt : gb;
  {
    unsigned g = 0, ti = 0;
    for (int64_t j0 = w0; j0 < w1; j0 += 64 * B) {
      unsigned key[B];
      batch(j0, key);
#pragma unroll
      for (int k = 0; k < B; ++k) {
        g += (unsigned)__popcll(__builtin_amdgcn_ballot_w64(key[k] != 0u && key[k] > T));
        ti += (unsigned)__popcll(__builtin_amdgcn_ballot_w64(key[k] != 0u && key[k] == T));
        const int64_t pos = j0 + 64 * (k + 1);   // positions covered so far
        if ((pos - w0) % kToprGroup == 0 || pos >= w1) {
          if (lane == 0) {
            const int64_t grp = (pos - 1 - (pos > w1 ? pos - w1 : 0)) / kToprGroup;
            cnt[2 * grp] = g;
            cnt[2 * grp + 1] = ti;
          }
          g = 0; ti = 0;
          if (pos >= w1) break;
        }
      }
    }
  }
  __syncthreads();
  // ---- exclusive scans over the groups: ties first (which ties are taken),
  // then records (greater + taken ties)
  {
    unsigned tie_base = 0, rec_base = 0;
    for (int64_t g0 = 0; g0 < ngroups; g0 += kToprThreads) {
      const int64_t gi = g0 + threadIdx.x;
      const unsigned gt = gi < ngroups ? cnt[2 * gi] : 0u;
      const unsigned ti = gi < ngroups ? cnt[2 * gi + 1] : 0u;
      int tot;
      const unsigned tp = (unsigned)block_excl_scan((int)ti, sh, &tot) + tie_base;
      const unsigned taken = tp >= need ? 0u : min(ti, need - tp);
      int tot2;
      const unsigned rp = (unsigned)block_excl_scan((int)(gt + taken), sh, &tot2) + rec_base;
      if (gi < ngroups) { gb[2 * gi] = rp; gb[2 * gi + 1] = tp; }   // after every read of cnt (scan barriers)
      tie_base += (unsigned)tot;
      rec_base += (unsigned)tot2;
    }
  }
}

// One wave per group of 1024 positions of a (unit, side), or of a unit's
// joint list (joint: positions (side * H + head) * N + token, both sides ranked
// together, the records numbered across both; the record list holds the
// side-inclusive position).
__global__ __launch_bounds__(256) void k_topr_flag(const float* util, const unsigned* groups, uint8_t* cache,
                                                   int64_t stride, int64_t off_words, int64_t off_ck, int64_t off_cv,
                                                   int* sel_list, int2* sel_aux, const int* aidx, const float* gam,
                                                   int Rmax, int H, int N, int C, int R, int US, int joint) {
  const int lane = threadIdx.x & 63;
  const int64_t M = (int64_t)(joint ? 2 * H : H) * N;
  const int64_t ngroups = (M + kToprGroup - 1) / kToprGroup;
  const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // over [US][ngroups]
  if (gw >= (int64_t)US * ngroups) return;
  const int us = (int)(gw / ngroups);
  const int64_t grp = gw - (int64_t)us * ngroups;
  const int u = joint ? us : us / 2, side_us = joint ? 0 : us % 2;
  int* chunk_k = reinterpret_cast<int*>(cache + (int64_t)u * stride + off_ck);
  int* chunk_v = reinterpret_cast<int*>(cache + (int64_t)u * stride + off_cv);
  const unsigned* tn = groups + (int64_t)US * ngroups * 2 + (int64_t)us * 2;
  const unsigned T = tn[0], need = tn[1];
  const unsigned rec_base = groups[((int64_t)us * ngroups + grp) * 2];
  const unsigned tie_base = groups[((int64_t)us * ngroups + grp) * 2 + 1];
  const float* up = util + (int64_t)us * M;
  const int* ap = aidx + (int64_t)us * M;
  const float* gp = gam + (int64_t)us * M;
  uint32_t* words = reinterpret_cast<uint32_t*>(cache + (int64_t)u * stride + off_words);
  const int64_t i0 = grp * kToprGroup;
  constexpr int S = kToprGroup / 64;
  float v[S], gv[S];
  int av[S];
#pragma unroll
  for (int k = 0; k < S; ++k) {
    const int64_t i = i0 + 64 * k + lane;
    v[k] = i < M ? up[i] : -1.0f;
    av[k] = i < M ? ap[i] : 0;
    gv[k] = i < M ? gp[i] : 0.0f;
  }
  unsigned run_tie = 0, run_sel = 0;
#pragma unroll
  for (int k = 0; k < S; ++k) {
    const int64_t i = i0 + 64 * k + lane;
    const unsigned key = R > 0 ? util_key(v[k]) : 0u;
    const bool gt = key != 0u && key > T;
    const bool tie = key != 0u && key == T;
    const unsigned long long mt = __builtin_amdgcn_ballot_w64(tie);
    const unsigned tie_rank = tie_base + run_tie + __builtin_amdgcn_mbcnt_hi((unsigned)(mt >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((unsigned)mt, 0u));
    const bool sel = gt || (tie && tie_rank < need);
    const unsigned long long ms = __builtin_amdgcn_ballot_w64(sel);
    const unsigned rec = rec_base + run_sel + __builtin_amdgcn_mbcnt_hi((unsigned)(ms >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((unsigned)ms, 0u));
    if (i < M) {
      const unsigned iu = (unsigned)i;   // 2*H*N < 2^31
      const int hr = (int)(iu / (unsigned)N), t = (int)(iu - (unsigned)hr * (unsigned)N);
      const int side = joint ? (hr >= H ? 1 : 0) : side_us;
      const int h = hr - (joint && side ? H : 0);
      if ((t & (kChunk - 1)) == 0) (side ? chunk_v : chunk_k)[h * C + t / kChunk] = (int)rec;
      const bool taken = sel && rec < (unsigned)R;
      // the token's pointer word: anchor index, residual flag, fp16 gamma
      words[((int64_t)h * N + t) * 2 + side] =
          (uint32_t)av[k] | (taken ? 0x8000u : 0u) | ((uint32_t)f2h_sat(gv[k]) << 16);
      if (taken) {
        sel_list[(int64_t)us * Rmax + rec] = hr * N + t;
        // the record's anchor and coefficient, so that the quantiser's loads
        // do not wait on the position first
        sel_aux[(int64_t)us * Rmax + rec] = make_int2(av[k], __float_as_int(gv[k]));
      }
    }
    run_tie += (unsigned)__popcll(mt);
    run_sel += (unsigned)__popcll(ms);
  }
}

// ------------------------------------------------------------ quantise+pack
// 16 lanes per residual record, 4 records per lane group in flight; lane j
// owns coordinates 8j..8j+7 (group j/4).  r = x - gamma x_a in f32 with the
// unrounded gamma; per 32-group: zero = fp16(min), scale = fp16((max-min)/3),
// code = clamp(rne((r - zero)/scale), 0, 3) (0 when scale = 0).  Record: code
// word j holds coordinates j + 16c in bits 2c..2c+1, then (scale, zero) x 4.
constexpr int kQuantPerGroup = 4;

// joint: one list of R records per unit over both sides (blocks per unit, not
// per (unit, side)); a record's side is in its position (side * H + head) * N + t.
template <int DT>
__global__ __launch_bounds__(256) void k_quant(const void* Kv, const void* Vv, uint8_t* cache, int64_t stride,
                                              int64_t off_ak, int64_t off_av, int64_t off_rk, int64_t off_rv,
                                              const int* sel_list, const int2* sel_aux, int Rmax, int H, int N, int A,
                                              int R, int nblk, int joint) {
  using T = typename Elem<DT>::T;
  constexpr int D = kHeadDim;
  constexpr int QG = kQuantPerGroup;
  __shared__ uint8_t codes_s[16][QG][128];
  int bid = blockIdx.x;
  const int blk = bid % nblk; bid /= nblk;
  const int side_b = joint ? 0 : bid % 2;
  const int u = joint ? bid : bid / 2;
  const int grp = threadIdx.x >> 4, j = threadIdx.x & 15;
  const int us = joint ? u : u * 2 + side_b;
  const int rec0 = (blk * 16 + grp) * QG;
  int flat[QG], a[QG], sd[QG];
  float g[QG];
#pragma unroll
  for (int k = 0; k < QG; ++k) {
    const bool act = rec0 + k < R;
    flat[k] = act ? sel_list[(int64_t)us * Rmax + rec0 + k] : 0;
    const int2 x = act ? sel_aux[(int64_t)us * Rmax + rec0 + k] : make_int2(0, 0);
    a[k] = x.x;
    g[k] = __int_as_float(x.y);
    sd[k] = joint ? (flat[k] >= H * N ? 1 : 0) : side_b;
    flat[k] -= joint && sd[k] ? H * N : 0;
  }
  float r[QG][8];
#pragma unroll
  for (int k = 0; k < QG; ++k) {
    const int side = sd[k];
    const int h = (int)((unsigned)flat[k] / (unsigned)N), t = flat[k] - h * N;
    const T* X = reinterpret_cast<const T*>(side ? Vv : Kv) + (((int64_t)u * H + h) * N + t) * D + 8 * j;
    const T* AX = reinterpret_cast<const T*>(cache + (int64_t)u * stride + (side ? off_av : off_ak)) +
                  ((int64_t)h * A + a[k]) * D + 8 * j;
    T xv[8], av[8];
    if constexpr (DT == ANCHORKV_BF16) {
      const uint4 x4 = *reinterpret_cast<const uint4*>(X), a4 = *reinterpret_cast<const uint4*>(AX);
      __builtin_memcpy(xv, &x4, 16);
      __builtin_memcpy(av, &a4, 16);
    } else {
      const uint4 x0 = *reinterpret_cast<const uint4*>(X), x1 = *reinterpret_cast<const uint4*>(X + 4);
      const uint4 a0 = *reinterpret_cast<const uint4*>(AX), a1 = *reinterpret_cast<const uint4*>(AX + 4);
      __builtin_memcpy(xv, &x0, 16); __builtin_memcpy(xv + 4, &x1, 16);
      __builtin_memcpy(av, &a0, 16); __builtin_memcpy(av + 4, &a1, 16);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) r[k][e] = fmaf(-g[k], Elem<DT>::f(av[e]), Elem<DT>::f(xv[e]));
  }
  uint16_t zb[QG], sb[QG];
#pragma unroll
  for (int k = 0; k < QG; ++k) {
    float mn = r[k][0], mx = r[k][0];
#pragma unroll
    for (int e = 1; e < 8; ++e) { mn = fminf(mn, r[k][e]); mx = fmaxf(mx, r[k][e]); }
    // the four lanes of a 32-coordinate group are one quad: DPP, no LDS
    mn = fminf(mn, dpp<kDppXor1>(mn)); mx = fmaxf(mx, dpp<kDppXor1>(mx));
    mn = fminf(mn, dpp<kDppXor2>(mn)); mx = fmaxf(mx, dpp<kDppXor2>(mx));
    zb[k] = f2h_sat(mn);
    sb[k] = f2h_sat((mx - mn) / 3.0f);
    const float z = h2f(zb[k]), sc = h2f(sb[k]);
    // one reciprocal per group: (r - z) * (1/sc) is within an ulp or two of
    // the quotient, which moves a code only next to a rounding boundary
    const float rinv = sc > 0.0f ? 1.0f / sc : 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float c = fminf(3.0f, fmaxf(0.0f, rintf((r[k][e] - z) * rinv)));
      codes_s[grp][k][8 * j + e] = (uint8_t)(int)c;
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < QG; ++k) {
    if (rec0 + k >= R) break;
    uint16_t wv = 0;
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) wv |= (uint16_t)(codes_s[grp][k][j + 16 * cc] << (2 * cc));
    // (joint: off_rv == off_rk and the record index counts across both sides)
    uint8_t* recp = cache + (int64_t)u * stride + (sd[k] ? off_rv : off_rk) + (int64_t)(rec0 + k) * kRecBytes;
    reinterpret_cast<uint16_t*>(recp)[j] = wv;
    // group q's (scale, zero) lives in lanes 4q..4q+3; lane 4q writes it
    if ((j & 3) == 0) reinterpret_cast<uint32_t*>(recp + 32)[j >> 2] = (uint32_t)sb[k] | ((uint32_t)zb[k] << 16);
  }
}

// The paper's codec (Pith review of AnchorKV, "Referee Report" summary and
// "Assumptions & free parameters": randomized Hadamard rotation with a fixed
// seed, 2-bit Lloyd-Max codebook for a unit Gaussian).  Per record, the 16
// lanes of a group hold coordinates 8j..8j+7: the residual is sign-flipped,
// Walsh-Hadamard transformed (three stages inside a lane, four across lanes:
// DPP for lane distances 1, 2 and 8, a swizzle for 4), and each coordinate
// of y / (sqrt(D) sigma) is compared with the thresholds -t, 0, t of the
// codebook; sigma = ||r|| / sqrt(D) in fp16.
constexpr float kLmThreshold = 0.98159882f;   // between the levels 0.45278 and 1.51042
__device__ __forceinline__ float swz_xor4(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x1F | (4 << 10)));
}
template <int DT>
__global__ __launch_bounds__(256) void k_quant_hlm(const void* Kv, const void* Vv, uint8_t* cache, int64_t stride,
                                                  int64_t off_ak, int64_t off_av, int64_t off_rk, int64_t off_rv,
                                                  const int* sel_list, const int2* sel_aux, int Rmax, int H, int N,
                                                  int A, int R, int nblk, int joint, uint4 signs) {
  using T = typename Elem<DT>::T;
  constexpr int D = kHeadDim;
  constexpr int QG = kQuantPerGroup;
  __shared__ uint8_t codes_s[16][QG][128];
  int bid = blockIdx.x;
  const int blk = bid % nblk; bid /= nblk;
  const int side_b = joint ? 0 : bid % 2;
  const int u = joint ? bid : bid / 2;
  const int grp = threadIdx.x >> 4, j = threadIdx.x & 15;
  const int us = joint ? u : u * 2 + side_b;
  const int rec0 = (blk * 16 + grp) * QG;
  const uint32_t sw = j < 4 ? signs.x : j < 8 ? signs.y : j < 12 ? signs.z : signs.w;
  const uint32_t sbyte = (sw >> (8 * (j & 3))) & 0xFFu;    // signs of coordinates 8j .. 8j+7
  int flat[QG], a[QG], sd[QG];
  float g[QG];
#pragma unroll
  for (int k = 0; k < QG; ++k) {
    const bool act = rec0 + k < R;
    flat[k] = act ? sel_list[(int64_t)us * Rmax + rec0 + k] : 0;
    const int2 x = act ? sel_aux[(int64_t)us * Rmax + rec0 + k] : make_int2(0, 0);
    a[k] = x.x;
    g[k] = __int_as_float(x.y);
    sd[k] = joint ? (flat[k] >= H * N ? 1 : 0) : side_b;
    flat[k] -= joint && sd[k] ? H * N : 0;
  }
  uint16_t sb[QG];
#pragma unroll
  for (int k = 0; k < QG; ++k) {
    const int side = sd[k];
    const int h = (int)((unsigned)flat[k] / (unsigned)N), t = flat[k] - h * N;
    const T* X = reinterpret_cast<const T*>(side ? Vv : Kv) + (((int64_t)u * H + h) * N + t) * D + 8 * j;
    const T* AX = reinterpret_cast<const T*>(cache + (int64_t)u * stride + (side ? off_av : off_ak)) +
                  ((int64_t)h * A + a[k]) * D + 8 * j;
    T xv[8], av[8];
    if constexpr (DT == ANCHORKV_BF16) {
      const uint4 x4 = *reinterpret_cast<const uint4*>(X), a4 = *reinterpret_cast<const uint4*>(AX);
      __builtin_memcpy(xv, &x4, 16);
      __builtin_memcpy(av, &a4, 16);
    } else {
      const uint4 x0 = *reinterpret_cast<const uint4*>(X), x1 = *reinterpret_cast<const uint4*>(X + 4);
      const uint4 a0 = *reinterpret_cast<const uint4*>(AX), a1 = *reinterpret_cast<const uint4*>(AX + 4);
      __builtin_memcpy(xv, &x0, 16); __builtin_memcpy(xv + 4, &x1, 16);
      __builtin_memcpy(av, &a0, 16); __builtin_memcpy(av + 4, &a1, 16);
    }
    float y[8];
    float ss = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float r = fmaf(-g[k], Elem<DT>::f(av[e]), Elem<DT>::f(xv[e]));
      ss = fmaf(r, r, ss);
      y[e] = (sbyte >> e) & 1u ? -r : r;
    }
    // scale: ||r|| / sqrt(D) in fp16
    ss = row_sum(ss);
    sb[k] = f2h_sat(sqrtf(ss) * 0.088388347648318f);
    // Walsh-Hadamard transform over i = 8j + e: bits 0-2 of i inside the lane
#pragma unroll
    for (int b = 1; b < 8; b <<= 1)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (!(e & b)) {
          const float p0 = y[e], p1 = y[e | b];
          y[e] = p0 + p1;
          y[e | b] = p0 - p1;
        }
    // bits 3-6 of i are bits 0-3 of the lane: the upper lane of a pair takes
    // partner - own, the lower own + partner
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float o = dpp<kDppXor1>(y[e]);
      y[e] = (j & 1) ? o - y[e] : y[e] + o;
      o = dpp<kDppXor2>(y[e]);
      y[e] = (j & 2) ? o - y[e] : y[e] + o;
      o = swz_xor4(y[e]);
      y[e] = (j & 4) ? o - y[e] : y[e] + o;
      o = dpp<kDppRor8>(y[e]);            // lane j + 8 mod 16 = lane j ^ 8
      y[e] = (j & 8) ? o - y[e] : y[e] + o;
    }
    const float sg = h2f(sb[k]);
    const float inv = sg > 0.0f ? 1.0f / (11.313708498984761f * sg) : 0.0f;   // 1 / (sqrt(D) sigma)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float uu = y[e] * inv;
      const int c = (uu >= -kLmThreshold ? 1 : 0) + (uu >= 0.0f ? 1 : 0) + (uu >= kLmThreshold ? 1 : 0);
      codes_s[grp][k][8 * j + e] = sg > 0.0f ? (uint8_t)c : (uint8_t)0;
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < QG; ++k) {
    if (rec0 + k >= R) break;
    uint16_t wv = 0;
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) wv |= (uint16_t)(codes_s[grp][k][j + 16 * cc] << (2 * cc));
    uint8_t* recp = cache + (int64_t)u * stride + (sd[k] ? off_rv : off_rk) + (int64_t)(rec0 + k) * kRecBytesHlm;
    reinterpret_cast<uint16_t*>(recp)[j] = wv;
    if (j == 0) *reinterpret_cast<uint32_t*>(recp + 32) = (uint32_t)sb[k];
  }
}

// (cos, sin) of the rotation angle t * base^(-2i/D) of every position t < N
// and pair i < D/2 (Pith review, "Assumptions & free parameters": RoPE as a
// per-position orthogonal map): angle and functions in double precision,
// rounded once to float.
__global__ __launch_bounds__(256) void k_rope_table(float2* cs, int N, double base) {
  constexpr int P = kHeadDim / 2;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)N * P) return;
  const int t = (int)(i / P), j = (int)(i % P);
  const double ang = (double)t * pow(base, -2.0 * j / kHeadDim);
  double sn, cn;
  sincos(ang, &sn, &cn);
  cs[i] = make_float2((float)cn, (float)sn);
}

// ------------------------------------------------------------ launch sequence
// Observation-window kernels on pre-RoPE keys: the generic kernels, with the
// keys (and in UTIL each token's anchor row) rotated while the tiles are
// staged; always 512 threads (the staging takes two items per thread; waves
// past the query blocks only stage).
// More than 8 query blocks (up to 16) take two workgroups per (unit, head,
// key split), each with 8 query blocks; their score (SCORE) and key-utility
// (UTIL) partials are added onto words zeroed here.
template <int DT, int MODE>
static int launch_obs_rope(const anchorkv_plan_info& p, const ObsArgs& a0, hipStream_t st) {
  const int QB = a0.GQp / 16;
  if (QB > 16) return fail(ANCHORKV_E_SHAPE, "pre-RoPE keys: q_per_kv*n_obs must be <= 256");
  ObsArgs a = a0;
  a.qsplit = QB > 8 ? 2 : 1;
  if (a.qsplit > 1 && MODE != OBS_STATS) {
    const int64_t H = p.H, N = p.N;
    // SCORE: score [U][H][N]; UTIL: the key side of util [U][2][H][N]
    unsigned* z = reinterpret_cast<unsigned*>(MODE == OBS_SCORE ? a.score : a.util);
    const int64_t len = MODE == OBS_SCORE ? (int64_t)p.units * H * N : H * N;
    const int64_t seg = MODE == OBS_SCORE ? len : 2 * H * N;
    const int64_t nseg = MODE == OBS_SCORE ? 1 : p.units;
    k_zero_seg<<<(unsigned)((len * nseg + 255) / 256), 256, 0, st>>>(z, len, seg, nseg);
    AKV_CHECK_LAUNCH("k_zero_seg");
  }
  const dim3 grid((unsigned)((int64_t)p.units * p.H * a.S1 * a.qsplit));
  // bf16: rotated keys as bf16 hi + lo on the bf16 MFMA; f32: f32 MFMA
  if constexpr (DT == ANCHORKV_BF16) k_obs<ANCHORKV_BF16, MODE, 1, ANCHORKV_BF16, true><<<grid, dim3(512), 0, st>>>(a);
  else k_obs<ANCHORKV_F32, MODE, 1, ANCHORKV_F32, true><<<grid, dim3(512), 0, st>>>(a);
  AKV_CHECK_LAUNCH("k_obs (pre-RoPE keys)");
  return 0;
}

template <int DT, int MODE>
static int launch_obs(const anchorkv_plan_info& p, const ObsArgs& a, hipStream_t st) {
  if (p.params.rope) return launch_obs_rope<DT, MODE>(p, a, st);
  const int QB = a.GQp / 16;
  int qpw = QB <= 8 ? 1 : 2;
  if (DT == ANCHORKV_F32 && QB > 8) return fail(ANCHORKV_E_SHAPE, "f32 path supports q_per_kv*n_obs <= 128");
  if (QB > 16) return fail(ANCHORKV_E_SHAPE, "q_per_kv*n_obs must be <= 256");
  const int nw = (QB + qpw - 1) / qpw;
  const dim3 block(64 * nw);
  if constexpr (DT == ANCHORKV_BF16) {
    const dim3 grid((unsigned)((int64_t)p.units * p.H * (MODE == OBS_UTIL ? a.S1u : a.S1)));
    using C1 = ObsPipeCfg<MODE, 1>;
    using C2 = ObsPipeCfg<MODE, 2>;
    if constexpr (MODE == OBS_UTIL) {
      // up to 6 query blocks: two key splits (12 waves, 3 per SIMD)
      const size_t qa_bytes = (size_t)((p.A + 15) / 16) * 16 * a.GQp * sizeof(float);
      if (qpw == 1 && nw <= 6 && qa_bytes <= kObsQaMaxBytes) {
        auto* fn = &k_obs_pipe<MODE, 1, C1::TK, C1::ST, 2, 3, true>;
        static size_t done = 0;
        if (int rc = set_dyn_lds(reinterpret_cast<const void*>(fn), qa_bytes, &done)) return rc;
        fn<<<grid, dim3(2 * 64 * nw), qa_bytes, st>>>(a);
      } else if (qpw == 1 && nw <= 6) k_obs_pipe<MODE, 1, C1::TK, C1::ST, 2, 3><<<grid, dim3(2 * 64 * nw), 0, st>>>(a);
      else if (qpw == 1) k_obs_pipe<MODE, 1, C1::TK, C1::ST, 1, 2><<<grid, block, 0, st>>>(a);
      else k_obs_pipe<MODE, 2, C2::TK, C2::ST, 1, 2><<<grid, block, 0, st>>>(a);
      // exact recompute of the tiles the fast pass flagged (its own stage)
      AKV_CHECK_LAUNCH("k_obs_pipe");
      prof_mark(st, "obs_util");
      if (qpw == 1) k_obs_pipe<OBS_UTILX, 1, kObsUtilTK, 1, 1, 2><<<grid, block, 0, st>>>(a);
      else k_obs_pipe<OBS_UTILX, 2, kObsUtilTK, 1, 1, 2><<<grid, block, 0, st>>>(a);
    } else {
      if (qpw == 1) k_obs_pipe<MODE, 1, C1::TK, C1::ST, 1, 2><<<grid, block, 0, st>>>(a);
      else k_obs_pipe<MODE, 2, C2::TK, C2::ST, 1, 2><<<grid, block, 0, st>>>(a);
    }
  } else {
    const dim3 grid((unsigned)((int64_t)p.units * p.H * a.S1));
    k_obs<DT, MODE, 1><<<grid, block, 0, st>>>(a);
  }
  AKV_CHECK_LAUNCH("k_obs");
  return 0;
}

// Nearest-anchor assignment, bf16: one LDS-resident launch when the anchors
// of a head fit, else parts folded with atomicMax and a projection pass.
static int launch_assign_bf16(const anchorkv_plan_info& p, const CompressWs& w, const ObsArgs& oa, const void* K,
                              const void* V, uint8_t* cache, uint8_t* ws, hipStream_t st) {
  const int U = p.units, H = p.H, N = p.N, A = p.A;
  AssignArgs g{};
  g.K = reinterpret_cast<const uint16_t*>(K);
  g.V = reinterpret_cast<const uint16_t*>(V);
  g.cache = cache; g.stride = p.unit_stride;
  g.off_anchor_k = p.off_anchor_k; g.off_anchor_v = p.off_anchor_v;
  g.anorm = reinterpret_cast<const float2*>(ws + w.anorm);
  g.anchor_of = oa.anchor_of;
  g.aidx = reinterpret_cast<int*>(ws + w.aidx);
  g.gam = reinterpret_cast<float*>(ws + w.gam);
  g.rn2 = reinterpret_cast<float*>(ws + w.rn2);
  g.vn2 = reinterpret_cast<float*>(ws + w.vn2);
  g.score = oa.score;
  g.util = oa.util;
  g.H = H; g.N = N; g.A = A;
  const int64_t hs = (int64_t)U * 2 * H;
  // 8-wave blocks, two per compute unit, when a part's anchors fit twice in
  // LDS; larger anchor sets are walked in the fewest equal parts of at most
  // kAssignPartMax anchors by 16-wave blocks (each part reload is a barrier,
  // a copy and a wait for the whole compute unit)
  const bool multi = A > kAssignResMax;
  const int nparts = multi ? (A + kAssignPartMax - 1) / kAssignPartMax : 1;
  g.part = multi ? (int)round_up((A + nparts - 1) / nparts, 16) : A;
  const int part_a = std::min(A, g.part);
  const bool w8 = !multi && 2 * assign_lds_bytes(part_a, 8) <= 160 * 1024;
  const int waves = w8 ? 8 : 16;
  const int ntiles_hs = (N + 64 * waves - 1) / (64 * waves);
  // tiles per block: fewest rounds of resident blocks times (tiles + a prologue
  // of about half a tile), larger runs on ties
  {
    const int64_t slots = 256 * (w8 ? 2 : 1);
    double best = 1e300;
    int tpb = 1;
    for (int c = 1; c <= ntiles_hs; ++c) {
      const int64_t grid_c = hs * ((ntiles_hs + c - 1) / c);
      const double cost = (double)((grid_c + slots - 1) / slots) * (c + 0.5);
      if (cost <= best) { best = cost; tpb = c; }
    }
    g.tiles_per_block = tpb;
    g.nblk = (ntiles_hs + tpb - 1) / tpb;
  }
  g.xcd_groups = 0;
  unsigned grid = (unsigned)(hs * g.nblk);
  if (A > kAssignResMax) {
    // anchors in parts reloaded every tile: the blocks of a (unit, side,
    // head) run together on one XCD (32 compute units) so that the reloads
    // hit its L2
    const int nb = 32;   // one block on each of the XCD's 32 compute units
    g.tiles_per_block = (ntiles_hs + nb - 1) / nb;
    g.nblk = (ntiles_hs + g.tiles_per_block - 1) / g.tiles_per_block;
    g.xcd_groups = (int)hs;
    const int64_t rounds = (hs + 7) / 8;
    grid = (unsigned)(rounds * 8 * g.nblk);
  }
  g.a0 = 0; g.a1 = A;
  if (A <= kAssignResMax) {
    const size_t lds = assign_lds_bytes(A, waves);
    if (w8) {
      static size_t done = 0;
      if (int rc = set_dyn_lds(reinterpret_cast<const void*>(&k_assign_res<false, 8>), lds, &done)) return rc;
      k_assign_res<false, 8><<<grid, 64 * 8, lds, st>>>(g);
    } else {
      static size_t done = 0;
      if (int rc = set_dyn_lds(reinterpret_cast<const void*>(&k_assign_res<false, 16>), lds, &done)) return rc;
      k_assign_res<false, 16><<<grid, 64 * 16, lds, st>>>(g);
    }
  } else {
    // the parts are walked inside the kernel (tokens read once)
    const size_t lds = assign_lds_bytes(g.part, 16);
    static size_t done = 0;
    if (int rc = set_dyn_lds(reinterpret_cast<const void*>(&k_assign_res<true, 16>), lds, &done)) return rc;
    k_assign_res<true, 16><<<grid, 64 * 16, lds, st>>>(g);
  }
  AKV_CHECK_LAUNCH("k_assign_res");
  return 0;
}

template <int DT>
static int compress_impl(const anchorkv_plan_info& p, const void* K, const void* V, const void* Q, void* cache_v,
                         void* ws_v, hipStream_t st) {
  uint8_t* cache = reinterpret_cast<uint8_t*>(cache_v);
  uint8_t* ws = reinterpret_cast<uint8_t*>(ws_v);
  const CompressWs w = compress_ws_layout(p);
  const int U = p.units, H = p.H, N = p.N, A = p.A, C = p.n_chunks;
  const int GQ = p.G * p.n_obs;
  if (A > 4096) return fail(ANCHORKV_E_SHAPE, "anchors per head %d > 4096 not supported", A);

  prof_call_begin(st);
  UnitHeader hd;
  fill_header(p, &hd);
  k_headers<<<U, 64, 0, st>>>(hd, cache, p.unit_stride);
  AKV_CHECK_LAUNCH("k_headers");

  ObsArgs a{};
  a.K = K; a.V = V; a.Q = Q; a.cache = cache; a.stride = p.unit_stride; a.off_anchor_k = p.off_anchor_k;
  a.ml_part = reinterpret_cast<float2*>(ws + w.ml_part);
  a.ml = reinterpret_cast<const float2*>(ws + w.ml);
  a.o_part = reinterpret_cast<float*>(ws + w.o_part);
  a.ohl = reinterpret_cast<const uint16_t*>(ws + w.ohl);
  a.ofull = reinterpret_cast<const float*>(ws + w.o);
  a.oo = reinterpret_cast<const float*>(ws + w.oo);
  a.score = reinterpret_cast<float*>(ws + w.score);
  a.gam = reinterpret_cast<const float*>(ws + w.gam);
  a.aidx = reinterpret_cast<const int*>(ws + w.aidx);
  a.rn2 = reinterpret_cast<const float*>(ws + w.rn2);
  a.anchor_of = reinterpret_cast<const int*>(ws + w.anchor_of);
  a.vn2 = reinterpret_cast<const float*>(ws + w.vn2);
  a.util = reinterpret_cast<float*>(ws + w.util);
  a.uflag = ws + w.uflag;
  a.nflag = (N + kObsUtilTK - 1) / kObsUtilTK;
  a.U = U; a.H = H; a.G = p.G; a.N = N; a.n_obs = p.n_obs; a.GQ = GQ; a.GQp = w.GQp; a.S1 = w.S1;
  a.kps = (int)round_up((N + w.S1 - 1) / w.S1, 64);
  a.S1u = std::max(w.S1, (N + kObsUtilMaxKeys - 1) / kObsUtilMaxKeys);
  a.kps_u = (int)round_up((N + a.S1u - 1) / a.S1u, 64);
  a.A = A;
  a.c = kLog2e / sqrtf((float)kHeadDim);
  a.inv_sqrt_d = 1.0f / sqrtf((float)kHeadDim);
  a.rope_cs = reinterpret_cast<const float2*>(ws + w.rope_cs);
  if (p.params.rope) {
    const int64_t n = (int64_t)N * (kHeadDim / 2);
    k_rope_table<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(reinterpret_cast<float2*>(ws + w.rope_cs), N,
                                                            (double)p.params.rope_theta);
    AKV_CHECK_LAUNCH("k_rope_table");
  }

  int rc;
  if ((rc = launch_obs<DT, OBS_STATS>(p, a, st))) return rc;
  prof_mark(st, "obs_stats");
  {
    const int64_t n = (int64_t)U * H * w.GQp;
    k_ml_combine<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(a.ml_part, reinterpret_cast<float2*>(ws + w.ml), w.S1,
                                                             w.GQp, GQ, n);
    AKV_CHECK_LAUNCH("k_ml_combine");
  }
  prof_mark(st, "ml_combine");
  if ((rc = launch_obs<DT, OBS_SCORE>(p, a, st))) return rc;
  prof_mark(st, "obs_score");
  k_o_combine<<<(unsigned)((int64_t)U * H * w.GQp), 128, 0, st>>>(
      a.o_part, reinterpret_cast<float*>(ws + w.o), reinterpret_cast<uint16_t*>(ws + w.ohl),
      reinterpret_cast<float*>(ws + w.oo), w.S1, w.GQp);
  AKV_CHECK_LAUNCH("k_o_combine");
  prof_mark(st, "o_combine");

  {
    // pooled score in LDS while it fits next to the static arrays (~26 KB)
    const size_t plb = sizeof(float) * (size_t)(N - p.window);
    const bool cover = p.params.anchor_mode == ANCHORKV_ANCHORS_COVER;
    int* clist = reinterpret_cast<int*>(ws + w.cover_list);
    auto sel = [&](auto kern, size_t dyn, int mode) {
      kern<<<(unsigned)(U * H), 1024, dyn, st>>>(
          K, V, a.score, reinterpret_cast<float*>(ws + w.pooled), cache, p.unit_stride, p.off_anchor_k,
          p.off_anchor_v, p.off_positions, reinterpret_cast<int*>(ws + w.anchor_of),
          reinterpret_cast<float2*>(ws + w.anorm), H, N, p.window, p.k_scored, p.k_uniform, A, p.params.pool, mode,
          clist);
    };
    // coverage anchors: scored positions (pass 1), the coverage picks, then
    // the final order, map and copies (pass 2)
    for (int pass = cover ? 1 : 0; pass <= (cover ? 2 : 0); ++pass) {
      if (pass == 2) {
        k_cover<DT><<<(unsigned)(U * H), 1024, 0, st>>>(K, clist, reinterpret_cast<float*>(ws + w.cover_mc), H, N,
                                                        p.window, p.k_scored, p.k_uniform, p.params.cover_rounds);
        AKV_CHECK_LAUNCH("k_cover");
      }
      if (N - p.window <= kSelectLdsMaxL) {
        static size_t sdone = 0;
        if ((rc = set_dyn_lds(reinterpret_cast<const void*>(&k_select<DT, true>), plb, &sdone))) return rc;
        sel(k_select<DT, true>, plb, pass);
      } else {
        sel(k_select<DT, false>, 0, pass);
      }
    }
  }
  AKV_CHECK_LAUNCH("k_select");
  prof_mark(st, "select");

  if constexpr (DT == ANCHORKV_BF16) {
    if ((rc = launch_assign_bf16(p, w, a, K, V, cache, ws, st))) return rc;
  } else {
    const int ntiles = (N + 255) / 256;
    k_assign<DT><<<(unsigned)((int64_t)U * 2 * H * ntiles), 256, 0, st>>>(
        K, V, cache, p.unit_stride, p.off_anchor_k, p.off_anchor_v,
        reinterpret_cast<const float2*>(ws + w.anorm), a.anchor_of, reinterpret_cast<int*>(ws + w.aidx),
        reinterpret_cast<float*>(ws + w.gam), reinterpret_cast<float*>(ws + w.rn2), reinterpret_cast<float*>(ws + w.vn2),
        a.score, a.util, H, N, A, ntiles);
    AKV_CHECK_LAUNCH("k_assign");
  }
  prof_mark(st, "assign");

  if ((rc = launch_obs<DT, OBS_UTIL>(p, a, st))) return rc;
  prof_mark(st, DT == ANCHORKV_BF16 && !p.params.rope ? "util_fix" : "obs_util");

  // top-R per (unit, side) with R_K == R_V, or per unit over both sides (joint)
  const bool joint = p.joint != 0;
  const int R = joint ? p.R_total : p.R_K;
  const int Rmax = (int)std::max<int64_t>(1, sel_stride(p));
  const int HS = joint ? 2 * H : H;           // rows of one ranking
  const int US = joint ? U : U * 2;           // rankings
  int* sel_list = reinterpret_cast<int*>(ws + w.sel_list);
  unsigned* groups = reinterpret_cast<unsigned*>(ws + w.sel_groups);
  if ((int64_t)HS * N <= (int64_t)kToprThreads * kToprKPT)
    k_topr_threshold<kToprKPT><<<(unsigned)US, kToprThreads, 0, st>>>(a.util, groups, HS, N, R);
  else
    k_topr_threshold<0><<<(unsigned)US, kToprThreads, 0, st>>>(a.util, groups, HS, N, R);
  AKV_CHECK_LAUNCH("k_topr_threshold");
  {
    const int64_t nw = (int64_t)US * (((int64_t)HS * N + kToprGroup - 1) / kToprGroup);
    k_topr_flag<<<(unsigned)((nw + 3) / 4), 256, 0, st>>>(a.util, groups, cache, p.unit_stride, p.off_words,
                                                          p.off_chunk_k, p.off_chunk_v, sel_list,
                                                          reinterpret_cast<int2*>(ws + w.sel_aux),
                                                          reinterpret_cast<const int*>(ws + w.aidx),
                                                          reinterpret_cast<const float*>(ws + w.gam), Rmax, H, N, C,
                                                          R, US, joint ? 1 : 0);
    AKV_CHECK_LAUNCH("k_topr_flag");
  }
  prof_mark(st, "topr");
  if (R > 0) {
    const int nblk = (R + 16 * kQuantPerGroup - 1) / (16 * kQuantPerGroup);
    if (p.params.codec == ANCHORKV_CODEC_HADAMARD_LM) {
      const uint4 sg = make_uint4(p.params.hadamard_signs[0], p.params.hadamard_signs[1], p.params.hadamard_signs[2],
                                  p.params.hadamard_signs[3]);
      k_quant_hlm<DT><<<(unsigned)((int64_t)US * nblk), 256, 0, st>>>(
          K, V, cache, p.unit_stride, p.off_anchor_k, p.off_anchor_v, p.off_res_k, p.off_res_v, sel_list,
          reinterpret_cast<const int2*>(ws + w.sel_aux), Rmax, H, N, A, R, nblk, joint ? 1 : 0, sg);
      AKV_CHECK_LAUNCH("k_quant_hlm");
    } else {
      k_quant<DT><<<(unsigned)((int64_t)US * nblk), 256, 0, st>>>(
          K, V, cache, p.unit_stride, p.off_anchor_k, p.off_anchor_v, p.off_res_k, p.off_res_v, sel_list,
          reinterpret_cast<const int2*>(ws + w.sel_aux), Rmax, H, N, A, R, nblk, joint ? 1 : 0);
      AKV_CHECK_LAUNCH("k_quant");
    }
  }
  prof_mark(st, "quant");
  return 0;
}

int compress_supports(const anchorkv_plan_info& p) {
  const int QB = padded_queries(p) / 16;
  if (p.dtype == ANCHORKV_F32 && QB > 8) return fail(ANCHORKV_E_SHAPE, "anchorkv_plan: f32 needs q_per_kv*n_obs <= 128");
  if (QB > 16) return fail(ANCHORKV_E_SHAPE, "anchorkv_plan: q_per_kv*n_obs must be <= 256");
  if (p.A > 4096) return fail(ANCHORKV_E_SHAPE, "anchorkv_plan: %d anchors per head; compress supports <= 4096", p.A);
  if (p.params.pool > kMaxPool) return fail(ANCHORKV_E_SHAPE, "anchorkv_plan: pool width > %d", kMaxPool);
  return 0;
}

int run_compress(const anchorkv_plan_info& p, const void* K, const void* V, const void* Q, void* cache, void* ws,
                 void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (p.dtype == ANCHORKV_BF16) return compress_impl<ANCHORKV_BF16>(p, K, V, Q, cache, ws, st);
  return compress_impl<ANCHORKV_F32>(p, K, V, Q, cache, ws, st);
}

}  // namespace akv
