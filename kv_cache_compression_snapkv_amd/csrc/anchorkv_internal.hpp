// Internal declarations shared by the host code and the HIP translation units.
#pragma once

#include <cstdint>
#include <cstddef>
#include <string>
#include <algorithm>

#include "anchorkv.h"

namespace akv {

constexpr int kHeaderBytes = 256;
constexpr int kChunk = 1024;          // tokens per residual-offset chunk
constexpr int kRecBytes = 48;         // group-affine residual record: 32 B codes + 4 x (fp16 scale, fp16 zero)
constexpr int kRecBytesHlm = 36;      // Hadamard / Lloyd-Max record: 32 B codes + fp16 scale + 2 zero bytes
inline int rec_bytes_of(int codec) { return codec == ANCHORKV_CODEC_HADAMARD_LM ? kRecBytesHlm : kRecBytes; }
inline int rec_bytes_of(const anchorkv_plan_info& p) { return rec_bytes_of(p.params.codec); }
constexpr int kGroup = 32;            // codec group (coordinates)
constexpr int kHeadDim = 128;         // the only supported head dim
constexpr uint32_t kMagic = 0x31564B41u;  // "AKV1"
constexpr int kMaxAnchors = 32767;
constexpr int kHistBins = 2048;       // radix-select digit bins (11 bits)
constexpr int kAssignResMax = 512;    // anchors per head held in LDS at once by the bf16 assignment
constexpr int kAssignPartMax = 576;   // larger sets: at most this many anchors per part (one block per compute unit)

void set_error(const char* fmt, ...);
int fail(int code, const char* fmt, ...);

inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Residual records of one unit (both sides) and the stride of the per-unit
// record lists of compress: per side, or both sides together when joint.
inline int64_t records_per_unit(const anchorkv_plan_info& p) {
  return p.joint ? (int64_t)p.R_total : (int64_t)p.R_K + p.R_V;
}
inline int64_t sel_stride(const anchorkv_plan_info& p) {
  return p.joint ? (int64_t)p.R_total : (int64_t)std::max(p.R_K, p.R_V);
}

// Splits of the key range per (unit, head) in the observation-window kernels.
int obs_splits(const anchorkv_plan_info& p);
inline int padded_queries(const anchorkv_plan_info& p) { return (int)round_up((int64_t)p.G * p.n_obs, 16); }

// Compress workspace layout (byte offsets from the workspace start).
struct CompressWs {
  int S1;          // key splits of the observation kernels
  int GQp;         // observation queries per KV head, padded to 16
  int64_t score;   // f32 [U][H][N]
  int64_t ml;      // float2 [U][H][GQp]   (m * log2(e)/sqrt(D), 1/l)
  int64_t o;       // f32 [U][H][GQp][D]
  int64_t util;    // f32 [U][2][H][N]
  int64_t gam;     // f32 [U][2][H][N]
  int64_t rn2;     // f32 [U][2][H][N]
  int64_t aidx;    // int32 [U][2][H][N]
  int64_t ml_part; // float2 [U][H][S1][GQp]
  int64_t o_part;  // f32 [U][H][S1][GQp][D]
  int64_t ohl;     // bf16 [U][H][2][GQp][D] (hi, lo split of o)
  int64_t oo;      // f32 [U][H][GQp] ||o||^2
  int64_t anchor_of; // int32 [U][H][N] anchor index of a position, -1 if none
  int64_t vn2;     // f32 [U][H][N] ||v_t||^2
  int64_t uflag;   // u8 [U][H][ceil(N/32)] utility tile flags (bf16 path)
  int64_t anorm;   // float2 [U][2][H][A] (||x_a||^2, 1/||x_a||)
  int64_t pooled;  // f32 [U][H][N]
  int64_t sel_list; // int32 [U][2][Rmax] flat (head*N + t) in record order
  int64_t sel_aux;  // (int32 anchor index, f32 unrounded gamma) [U][2][Rmax] in record order
  int64_t sel_groups; // u32 [U][2][ceil(H*N/1024)][2] record / tie bases per 1024 positions, then [U][2][2] (T, need)
  // coverage anchors only (params.anchor_mode == ANCHORKV_ANCHORS_COVER, else empty):
  int64_t cover_mc;   // f32 [U][H][N] largest cosine of each position to the anchors so far (+inf: an anchor)
  int64_t cover_list; // int32 [U][H][k_s + k_u] scored positions (ascending), then the picks in round order
  // pre-RoPE keys only (params.rope == 1, else empty):
  int64_t rope_cs;    // float2 [N][64] (cos, sin) of t * rope_theta^(-2i/128)
  int64_t total;
};
CompressWs compress_ws_layout(const anchorkv_plan_info& p);

// Decode workspace layout.
struct DecodeWs {
  int S2;          // token splits per (unit, head); boundaries on 1024-token chunks
  int64_t part_ml; // float2 [U][H][S2][G]  (max, sum) of each range
  int64_t part_acc; // f32 [U][H][S2][G][D] unnormalised output of each range
  int St;           // ranges per (unit, head) of an appended exact tail
  int64_t tail_ml;  // float2 [U][H][St][G] (max, sum) of each tail range
  int64_t tail_acc; // f32 [U][H][St][G][D] unnormalised output of each tail range
  int64_t total;
};
DecodeWs decode_ws_layout(const anchorkv_plan_info& p);

// Device header written at the start of every unit (256 bytes).
struct UnitHeader {
  uint32_t magic, version;
  int32_t H, G, N, D, n_obs, dtype, window;
  float theta;
  int32_t A, k_scored, k_uniform, R_K, R_V, n_chunks;
  int64_t off_anchor_k, off_anchor_v, off_res_k, off_res_v, off_words, off_chunk_k, off_chunk_v, off_positions;
  int64_t unit_bytes, unit_stride;
  int32_t unit_index, pad0;
  // the method's fixed parameters the unit was compressed with
  int32_t anchor_div, pool, group, pool_kv_jointly;
  double rho;
  int32_t R_total, pad1;   // joint ranking: residual records of both sides
  int32_t codec;           // residual codec (anchorkv_codec)
  uint32_t signs[4];       // rotation signs of the Hadamard / Lloyd-Max codec
  int32_t rope;            // 1: keys stored pre-RoPE, rotated at decode
  float rope_theta;        // rotary base of those keys
  uint8_t pad[256 - 16 * 4 - 10 * 8 - 8 - 4 * 4 - 8 - 8 - 4 - 16 - 8];
};
static_assert(sizeof(UnitHeader) == 256, "header must be 256 bytes");
void fill_header(const anchorkv_plan_info& p, UnitHeader* h);

// Stage profiler (HIP events between stages; off unless enabled).
void prof_call_begin(void* stream);
void prof_mark(void* stream, const char* stage);

// Launch sequences (defined in the HIP translation units).
int run_compress(const anchorkv_plan_info& p, const void* K, const void* V, const void* Q, void* cache,
                 void* ws, void* stream);
int run_decode(const anchorkv_plan_info& p, const void* cache, const void* q, float* o, void* ws, void* stream);
// Decode with an exact tail of n_tail tokens per KV head appended after the
// compressed ones: K_tail / V_tail [U][H][tail_cap][D] in the cache dtype.
int run_decode_tail(const anchorkv_plan_info& p, const void* cache, const void* q, const void* K_tail,
                    const void* V_tail, int n_tail, int tail_cap, float* o, void* ws, void* stream);
// Decode with its workspace in a static device array (no allocation by the
// caller or the library); at most kStaticScratchBytes of workspace.
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;
int run_decode_noalloc(const anchorkv_plan_info& p, const void* cache, const void* q, float* o, void* stream);
// Workgroups of the decode kernel that fit one compute unit (LDS and registers).
int decode_blocks_per_cu(int G, int A, bool f32, int codec);
// Host-only checks (no HIP calls) that the kernels can run a plan: 0, or a
// negative code with the message set.  anchorkv_plan refuses what fails them.
int compress_supports(const anchorkv_plan_info& p);
int decode_supports(const anchorkv_plan_info& p);
constexpr int kMaxPool = 15;          // widest positional pooling of the anchor score

}  // namespace akv
