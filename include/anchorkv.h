/*
 * anchorkv.h - C ABI of the anchor-residual KV-cache hot path (AnchorKV) on
 * AMD Instinct MI355X (gfx950).
 *
 * The method (web pages: "Pith review of AnchorKV: Anchor-Residual KV Cache
 * Compression", section "What carries the argument"; "AnchorKV-adapted -
 * Anchor-Residual Compression, No Eviction", sections "The problem this
 * solves" and "Adaptation notes") keeps a few anchor vectors per KV head
 * exactly and stores every other token as (anchor index a, coefficient gamma,
 * optional 2-bit residual), x^ = gamma * x_a + r~.  It runs once at the end of
 * prefill (compress) and decode attention then reads the compressed cache
 * directly (decode_attn).
 *
 * Conventions (all entry points):
 *  - Return 0 on success or a negative ANCHORKV_E_* code; anchorkv_last_error()
 *    then gives a message (thread-local, valid until the next call on the
 *    same thread).  Errors are found synchronously (argument checks, launch
 *    errors); a device fault surfaces at the caller's next synchronisation.
 *  - Device buffers are allocated and owned by the caller.  The library never
 *    allocates or frees device memory and never synchronises: everything is
 *    enqueued on `stream` (a hipStream_t; NULL = the default stream).
 *  - A "unit" is one layer of one sequence: H KV heads of N tokens.  Units are
 *    independent; the residual budget is pooled over the H heads of a unit.
 *  - Supported: head_dim == 128, dtype bf16 or f32, 1 <= window <= n_tokens,
 *    1 <= n_obs <= n_tokens, q_per_kv <= 8, anchors per head <= 4096 (see
 *    anchorkv_plan for the full list; the plan refuses what the kernels cannot run).
 *  - Inputs must be finite, with |x| small enough that residual scales and
 *    zeros fit fp16 (|x| < 1e4 is ample).
 */
#ifndef ANCHORKV_H
#define ANCHORKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  ANCHORKV_OK = 0,
  ANCHORKV_E_ARG = -1,          /* null pointer or invalid argument */
  ANCHORKV_E_DTYPE = -2,        /* unsupported dtype */
  ANCHORKV_E_SHAPE = -3,        /* unsupported shape */
  ANCHORKV_E_BUDGET = -4,       /* theta too small for the window anchors and the pointers */
  ANCHORKV_E_SMALL_BUFFER = -5, /* cache / workspace / output buffer too small */
  ANCHORKV_E_HIP = -6,          /* a HIP launch or runtime call failed */
  ANCHORKV_E_LAYOUT = -7        /* a cache header that does not describe a valid cache */
};

typedef enum { ANCHORKV_BF16 = 1, ANCHORKV_F32 = 2 } anchorkv_dtype;

/* Shapes.  K and V are [units][kv_heads][n_tokens][head_dim]; the observation
 * queries are [units][kv_heads*q_per_kv][n_obs][head_dim] (q-head h*q_per_kv+g
 * belongs to KV head h); decode queries are [units][kv_heads*q_per_kv][head_dim]. */
typedef struct {
  int32_t units;
  int32_t kv_heads;
  int32_t q_per_kv;
  int32_t n_tokens;
  int32_t head_dim;
  int32_t n_obs;
  int32_t dtype; /* anchorkv_dtype */
} anchorkv_dims;

/* The method's parameters (Pith review of AnchorKV, "Assumptions & free
 * parameters": theta the byte budget, W the recency window, k = S/128
 * non-window anchors, rho = 0.7 of them picked by the observation score,
 * positional pooling of width kappa = 7; AnchorKV-adapted page, "The one
 * setting worth tuning": theta is the only knob a user is meant to turn).
 * Fill with anchorkv_params_default, then change fields as needed. */
typedef struct {
  float theta;             /* bytes per side kept: floor(theta*H*N*D*e) per unit (0 < theta <= 1024) */
  int32_t window;          /* last `window` positions are always anchors (1 <= window <= n_tokens) */
  int32_t anchor_div;      /* non-window anchors k = floor(N / anchor_div), capped by the budget (>= 1; 128) */
  int32_t pool;            /* width of the positional pooling of the score (odd, 1..15; 7) */
  double rho;              /* k_scored = floor(rho * k) in double precision, the rest picked uniformly ([0, 1]; 0.7) */
  int32_t group;           /* group-affine codec: one fp16 scale and zero per `group` coordinates (32 only) */
  int32_t pool_kv_jointly; /* 0: separate residual budgets for K and V; 1: one ranking of all (side, head,
                              token) items under both sides' budgets together (0) */
  int32_t codec;           /* residual codec: ANCHORKV_CODEC_AFFINE (default) or ANCHORKV_CODEC_HADAMARD_LM */
  uint32_t hadamard_signs[4]; /* ANCHORKV_CODEC_HADAMARD_LM: rotation signs, bit i (bit i%32 of word i/32)
                                 set means coordinate i is negated before the transform; the default is
                                 the first two SplitMix64 outputs from seed 0x416E63686F724B56, low word
                                 first (Steele, Lea and Flood 2014) */
  int32_t anchor_mode;     /* the k_uniform non-scored anchors: ANCHORKV_ANCHORS_UNIFORM (default) or
                              ANCHORKV_ANCHORS_COVER */
  int32_t cover_rounds;    /* ANCHORKV_ANCHORS_COVER: rounds of the picks (1..1024; 8); with
                              cover_rounds >= k_uniform every round adds one anchor */
  int32_t rope;            /* 0: K holds the keys as attended (default); 1: K holds pre-RoPE keys and
                              the library applies the rotary embedding wherever a key meets a query
                              (see below) */
  float rope_theta;        /* rope = 1: rotary base (1 < rope_theta <= 1e10; 500000) */
  int32_t reserved[2];     /* zero */
} anchorkv_params;

/* Pre-RoPE key storage (rope = 1; Pith review of AnchorKV, "Assumptions &
 * free parameters": RoPE is a per-position orthogonal linear map R_t, so
 * R_t K_t = R_t K~_t + R_t r_t with ||R_t r_t|| = ||r_t||; "Referee Report":
 * pre-RoPE key storage with RoPE distributing over the decomposition).  R_t
 * turns coordinate pairs (i, i + 64) by the angle t * rope_theta^(-2i/128),
 * the key at position t (0-based).  Compress: the observation-window
 * attention, the anchor score and the key utility see the rotated keys (the
 * residual rotated at the token's position); anchors, nearest-anchor
 * assignment, gamma and residuals are those of the stored pre-RoPE keys.
 * Decode: logits <q, R_t(gamma k_a + r~)>/sqrt(D) with q given already
 * rotated; an appended tail is attended as given (its keys already rotated).
 * Needs the group-affine codec.  With more than 128 observation queries per
 * KV head (q_per_kv * n_obs up to 256) the observation passes give each
 * (unit, head, key range) two workgroups of up to 128 queries whose score and
 * key-utility partials are added. */

/* How the non-scored anchors are picked.  UNIFORM: stratified over the
 * positions left after the scored ones.  COVER: coverage-optimised (Pith
 * review of AnchorKV, "Reading between the lines": anchors placed for
 * coverage, by k-means or furthest-point picks), furthest-point sampling on
 * the keys in cover_rounds batched rounds: starting from the scored and window
 * anchors, round r adds the floor(k_u (r+1)/R) - floor(k_u r/R) non-window
 * positions that are not anchors yet with the lowest largest signed cosine to
 * the current anchors (0 where a norm is 0), the lower position on ties.
 * Counts and layout do not depend on the mode; decode does not read it. */
typedef enum { ANCHORKV_ANCHORS_UNIFORM = 0, ANCHORKV_ANCHORS_COVER = 1 } anchorkv_anchor_mode;

/* Residual codecs.  AFFINE: 2-bit codes with an fp16 scale and zero per 32
 * coordinates (48-byte records at head_dim 128).  HADAMARD_LM, the paper's
 * codec (Pith review of AnchorKV, "Referee Report" summary and "Assumptions &
 * free parameters": randomized Hadamard rotation with a fixed seed, 2-bit
 * Lloyd-Max codebook for a unit Gaussian): y = (1/sqrt(D)) H_D diag(s) r with
 * the Sylvester Hadamard matrix, one fp16 scale sigma = ||r||/sqrt(D) per
 * residual, code of y_i/sigma against the thresholds -t, 0, t (t = 0.9815988,
 * a value on a threshold takes the upper cell), levels -1.5104176, -0.4527800,
 * 0.4527800, 1.5104176; r~ = diag(s) (1/sqrt(D)) H_D (sigma * level[code])
 * (36-byte records). */
typedef enum { ANCHORKV_CODEC_AFFINE = 0, ANCHORKV_CODEC_HADAMARD_LM = 1 } anchorkv_codec;

/* Everything the host needs about a compressed cache: counts, byte accounting
 * and the per-unit layout.  Filled by anchorkv_plan or anchorkv_plan_from_header. */
typedef struct {
  /* shape and knobs */
  int32_t units, H, G, N, D, n_obs, dtype, elem_bytes, window;
  float theta;
  anchorkv_params params;  /* as passed to anchorkv_plan (theta and window repeated above) */
  /* counts per head / per unit (Pith review, "Assumptions & free parameters":
   * k = S/128 non-window anchors, rho = 0.7 scored, window W) */
  int32_t A;          /* anchors per head = window + k_scored + k_uniform */
  int32_t k_scored;   /* anchors picked by the pooled observation-window score */
  int32_t k_uniform;  /* anchors picked uniformly over the remaining positions */
  int32_t R_K, R_V;   /* residual slots per unit for keys / values (separate budgets; with joint
                       * ranking the slots of each side's budget alone, for reference) */
  int32_t n_chunks;   /* ceil(N / 1024): residual-offset chunks per head */
  /* byte accounting per side per unit (anchors D*e, pointers 4, residual D/4+D/8) */
  int64_t budget_bytes_per_side; /* floor(theta * H * N * D * e) */
  int64_t used_bytes_k, used_bytes_v;
  double compression_ratio;      /* 2*H*N*D*e / unit_bytes */
  /* per-unit cache layout: byte offsets from the start of a unit */
  int64_t off_anchor_k, off_anchor_v; /* [H][A][D] input dtype, stored exactly */
  int64_t off_res_k, off_res_v;       /* [R][48 or 36] residual records, sorted by (head, position); joint:
                                       * one section of R_total records, all key records first, then
                                       * the value records (off_res_v == off_res_k, and the value
                                       * chunk offsets count from the section start) */
  int64_t off_words;                  /* [H][N][2] uint32: K word, V word per token */
  int64_t off_chunk_k, off_chunk_v;   /* [H][n_chunks] int32: first record of each 1024-token chunk */
  int64_t off_positions;              /* [H][A] int32 anchor positions, ascending */
  int64_t unit_bytes;                 /* bytes of one unit's content */
  int64_t unit_stride;                /* unit_bytes rounded up to 16 */
  int64_t cache_bytes;                /* units * unit_stride */
  /* device scratch the caller provides */
  int64_t compress_workspace_bytes;
  int64_t decode_workspace_bytes;
  int32_t decode_splits;              /* token splits per (unit, head) in decode */
  int32_t joint;                      /* params.pool_kv_jointly */
  int32_t R_total;                    /* joint: residual records per unit, both sides together */
  int32_t reserved[5];
} anchorkv_plan_info;

/* Pointer word (uint32, one per token per side): bits 0-14 anchor index,
 * bit 15 set when the token has a residual record, bits 16-31 fp16 gamma.
 * Residual record, group-affine codec (48 bytes): 16 little-endian uint16 code
 * words, then 4 x (fp16 scale, fp16 zero) for the 32-coordinate groups.  Code
 * word j holds the 2-bit codes of coordinates j + 16c (c = 0..7) in bits
 * 2c..2c+1; group g is coordinates 32g..32g+31; the value is zero_g +
 * scale_g * code.  Hadamard / Lloyd-Max codec (36 bytes): the same 16 code
 * words over the rotated coordinates, then the fp16 scale sigma and two zero
 * bytes. */

/* Library version string. */
const char* anchorkv_version(void);

/* Message for the last non-zero return on this thread. */
const char* anchorkv_last_error(void);

/* Defaults of the method's fixed parameters (anchor_div 128, rho 0.7, pool 7,
 * group 32, separate K/V budgets, group-affine codec, the default rotation
 * signs) with the given theta and window.  Null is ignored. */
void anchorkv_params_default(anchorkv_params* params, float theta, int32_t window);

/* Counts, byte accounting and layout for (dims, params).  Host only, no HIP
 * calls.  Budget (per KV head and side) B = theta*N*D*e bytes with theta taken
 * at float32 precision; anchors A = window + min(N/anchor_div, A_max - window,
 * N - window) where A_max is the number of exact anchors the budget pays for
 * after pointers, chunk offsets and header; k_scored = floor(rho*(A - window));
 * residual slots per side per unit
 * R = min(H*(N-A), floor((floor(theta*H*N*D*e) - fixed)/rec)) with rec the
 * record size of the codec (D/4+D/8, or D/4+4 for the Hadamard / Lloyd-Max codec).
 * (Pith review, "What carries the argument" and "Assumptions & free
 * parameters"; AnchorKV-adapted page, "The one setting worth tuning".)
 * A shape that compress or decode cannot run is refused here: more than 4096
 * anchors per head, q_per_kv > 8, q_per_kv*n_obs > 256 (128 for f32), or a
 * decode working set (anchor logits and weights of q_per_kv q-heads) beyond
 * the 160 KB of LDS.
 * Errors: E_ARG (null, parameters out of range), E_DTYPE, E_SHAPE, E_BUDGET. */
int anchorkv_plan(const anchorkv_dims* dims, const anchorkv_params* params, anchorkv_plan_info* out);

/* Rebuild the plan from a host copy of a unit's first 256 bytes (the header
 * compress writes at the start of every unit; it records dims and params).
 * Errors: E_ARG, E_LAYOUT. */
int anchorkv_plan_from_header(const void* header_host, int32_t units, anchorkv_plan_info* out);

/* Section offsets of one unit of a compressed cache (bytes from the unit's
 * start), read from a host copy of its 256-byte header: for inspection and for
 * tools that read the cache without the plan. */
typedef struct {
  int64_t off_anchor_k, off_anchor_v, off_res_k, off_res_v, off_words, off_chunk_k, off_chunk_v, off_positions;
  int64_t unit_bytes, unit_stride;
  int32_t A, R_K, R_V, n_chunks, record_bytes, reserved[3];
} anchorkv_layout;
int anchorkv_cache_layout(const void* header_host, anchorkv_layout* out);

/* Decode workspace bytes for `units` units of the cache whose header (host
 * copy) is given: what anchorkv_decode_attn needs.  Errors: E_ARG, E_LAYOUT. */
int anchorkv_decode_workspace_bytes(const void* header_host, int32_t units, size_t* out);

/* End-of-prefill compression of all units (Pith review, "What carries the
 * argument"; AnchorKV-adapted page, "Adaptation notes": one pass, no
 * calibration).  Per unit and KV head: causal observation-window attention of
 * the n_obs last queries, pooled score (width 7), anchors = window + top
 * scored + uniform picks; per side, nearest anchor by cosine (lowest index on
 * ties, anchors map to themselves), gamma = <x, x_a>/||x_a||^2 stored fp16,
 * residual r = x - gamma x_a; first-order output-error utilities (key channel
 * p |<q, r_K>|/sqrt(D) ||v - o||, value channel p ||r_V||, summed over the
 * observation queries); the R_K / R_V largest utilities per unit get a 2-bit
 * residual record (ties: lower head, then lower position).
 *  K, V:    device, [units][H][N][D], dtype of the plan.
 *  Q_obs:   device, [units][H*G][n_obs][D]; query j of a q-head sits at
 *           position N - n_obs + j (causal).
 *  cache:   device, >= plan->cache_bytes, written completely.
 *  workspace: device, >= plan->compress_workspace_bytes; its contents after
 *           the call hold the intermediate arrays (see anchorkv_workspace_offsets).
 * The result is bitwise deterministic for given inputs.
 * Errors: E_ARG, E_SMALL_BUFFER, E_HIP. */
int anchorkv_compress(const anchorkv_plan_info* plan, const void* K, const void* V, const void* Q_obs,
                      void* cache, size_t cache_bytes, void* workspace, size_t workspace_bytes,
                      void* stream);

/* Offsets (bytes from the workspace start) of compress intermediates, for
 * inspection in tests: [0] score f32 [U][H][N]; [1] m,1/l float2 [U][H][GQp];
 * [2] o f32 [U][H][GQp][D]; [3] utilities f32 [U][2][H][N] (-1 for anchors);
 * [4] unrounded gamma f32 [U][2][H][N]; [5] residual norm^2 f32 [U][2][H][N]
 * (value side; the key half is 0 for bf16 caches);
 * [6] anchor index int32 [U][2][H][N].  out[7] = GQp, the number of
 * observation queries per KV head (q_per_kv * n_obs) rounded up to a multiple
 * of 16; query row g*n_obs + j is q-head g, observation j.  Returns 0 or E_ARG. */
int anchorkv_workspace_offsets(const anchorkv_plan_info* plan, int64_t out[8]);

/* Decode attention over the compressed cache, one query per q-head per unit
 * (Pith review, "What carries the argument": logits gamma*<q, k_a> + <q, r~>,
 * values reconstructed the same way; softmax over all N compressed tokens,
 * no mask).  The dense cache is never materialised.
 *  plan:   host; the plan the cache was written with (anchorkv_plan, or
 *          anchorkv_plan_from_header on a host copy of the first unit's
 *          header).  The launch shape depends on it, and reading it from the
 *          device cache would cost a device-to-host copy and a wait per call,
 *          which the library never does.  Instead every workgroup checks its
 *          unit's header on the device against the plan (magic, H, N, A, R_K,
 *          R_V, unit size) and, on a mismatch, writes NaN to that unit's
 *          outputs without reading the rest of the unit.
 *  cache:  device, >= plan->cache_bytes (cache_bytes is checked), as written
 *          by anchorkv_compress or packed on the host.
 *  q:      device, [units][H*G][D], cache dtype.
 *  o:      device, [units][H*G][D] float32.
 *  workspace: device, >= plan->decode_workspace_bytes.
 * Errors: E_ARG, E_SMALL_BUFFER, E_HIP. */
int anchorkv_decode_attn(const anchorkv_plan_info* plan, const void* cache, size_t cache_bytes, const void* q,
                         float* o, void* workspace, size_t workspace_bytes, void* stream);

/* Decode attention exactly as anchorkv_decode_attn, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): no workspace argument.  The workspace
 * lives in a static device array of 16 MiB that each GPU the library runs on
 * holds until the process ends; its device address is looked up once per
 * device.  Plans that need more decode workspace than that (more than about
 * 16 MiB of per-range partials: units * kv_heads * splits * q_per_kv * 520
 * bytes) are refused with E_SMALL_BUFFER.  Every call on a GPU shares that
 * GPU's array: calls that overlap on one GPU (other streams, other threads)
 * race and must be serialised by the caller.  The library allocates and
 * frees nothing here.
 * Errors: E_ARG, E_SMALL_BUFFER (cache too small, or the plan's workspace
 * exceeds the static array), E_HIP. */
int anchorkv_decode_attn_noalloc(const anchorkv_plan_info* plan, const void* cache, size_t cache_bytes, const void* q,
                                 float* o, void* stream);

/* Decode attention over the compressed cache followed by a tail of tokens
 * appended after the one-shot compression and kept uncompressed
 * (AnchorKV-adapted page, "Adaptation notes": tokens produced during decode
 * are appended at full precision and never re-anchored).  Each q-head takes
 * one softmax over the N compressed tokens and the n_tail tail tokens of its
 * KV head.
 *  K_tail, V_tail: device, [units][H][tail_cap][D], cache dtype, 16-byte
 *           aligned; rows [0, n_tail) of every head are read.  The same n_tail
 *           applies to every unit.  May be null when n_tail = 0.
 *  n_tail = 0 runs exactly the launches of anchorkv_decode_attn.
 *  The other arguments are those of anchorkv_decode_attn (same workspace).
 * Errors: E_ARG (null or misaligned buffers, n_tail < 0, n_tail > tail_cap),
 *         E_SMALL_BUFFER, E_HIP. */
int anchorkv_decode_attn_tail(const anchorkv_plan_info* plan, const void* cache, size_t cache_bytes, const void* q,
                              const void* K_tail, const void* V_tail, int32_t n_tail, int32_t tail_cap, float* o,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Host-side view of one unit's compressed representation, as plain arrays.
 * All pointers are host memory owned by the caller. */
typedef struct {
  int32_t* positions;  /* [H][A] anchor positions, ascending */
  void* anchors_k;     /* [H][A][D] cache dtype */
  void* anchors_v;     /* [H][A][D] */
  int32_t* idx;        /* [2][H][N] anchor index (side 0 = K, 1 = V) */
  uint16_t* gamma16;   /* [2][H][N] fp16 bits of gamma */
  uint8_t* flag;       /* [2][H][N] 1 if the token has a residual */
  uint8_t* codes;      /* [2][H][N][D] 2-bit codes (0..3); read/written only where flag */
  uint16_t* scale16;   /* [2][H][N][D/32] fp16 bits; only where flag (Hadamard / Lloyd-Max codec:
                          entry 0 of a token is its scale sigma, the others are 0) */
  uint16_t* zero16;    /* [2][H][N][D/32] fp16 bits; only where flag (0 for the Hadamard / Lloyd-Max codec) */
} anchorkv_unit_arrays;

/* Write one unit (plan->unit_bytes bytes, header included) into host memory
 * `unit_out` from plain arrays: the reference packer used by the tests and by
 * tools that build a cache outside compress.  Residual records are laid out
 * in (head, position) order; counts must equal plan->R_K / R_V.
 * Errors: E_ARG, E_LAYOUT (flag counts differ from the plan, index >= A). */
int anchorkv_unit_pack_host(const anchorkv_plan_info* plan, const anchorkv_unit_arrays* in, void* unit_out);

/* Inverse of anchorkv_unit_pack_host: decode one unit's bytes (host copy) into
 * plain arrays.  Errors: E_ARG, E_LAYOUT (bad header or inconsistent records). */
int anchorkv_unit_unpack_host(const anchorkv_plan_info* plan, const void* unit_in, anchorkv_unit_arrays* out);

/* Stage profiling for benchmarks (not part of the method).  When enabled,
 * every compress / decode call records a HIP event on its stream before its
 * first kernel and after each stage; anchorkv_profile_read waits for the last
 * recorded event and returns, per stage in call order, its name and elapsed
 * milliseconds, then clears the record.  Up to 1024 events are kept; stages
 * beyond that are not recorded.  Global state: enable, run and read from one
 * thread.  Errors: E_ARG, E_HIP. */
int anchorkv_profile_enable(int enable);
int anchorkv_profile_read(const char** names, float* ms, int max_stages, int* n_stages);

#ifdef __cplusplus
}
#endif

#endif /* ANCHORKV_H */
