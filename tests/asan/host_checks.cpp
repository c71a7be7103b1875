// Host-side checks of the C ABI's plan / layout / pack / unpack code under
// AddressSanitizer and UndefinedBehaviorSanitizer (built with g++, no HIP):
// many valid and invalid shapes and parameters, pack -> unpack round trips
// with residual records, headers rebuilt and corrupted.  The device launch
// sequences are replaced by stubs (they are never called here); the
// kernels' own host-side limits are replaced by permissive ones.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "anchorkv_internal.hpp"

namespace akv {
void prof_call_begin(void*) {}
void prof_mark(void*, const char*) {}
int run_compress(const anchorkv_plan_info&, const void*, const void*, const void*, void*, void*, void*) { return 0; }
int run_decode(const anchorkv_plan_info&, const void*, const void*, float*, void*, void*) { return 0; }
int run_decode_tail(const anchorkv_plan_info&, const void*, const void*, const void*, const void*, int, int, float*,
                    void*, void*) { return 0; }
int run_decode_noalloc(const anchorkv_plan_info&, const void*, const void*, float*, void*) { return 0; }
int decode_blocks_per_cu(int, int, bool, int) { return 1; }
int compress_supports(const anchorkv_plan_info&) { return 0; }
int decode_supports(const anchorkv_plan_info&) { return 0; }
}  // namespace akv

static int failures = 0;
#define CHECK(c)                                                      \
  do {                                                                \
    if (!(c)) {                                                       \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

// one unit with every eligible (side, head, token) flagged in order until the plan's counts
static void roundtrip(const anchorkv_plan_info& p, std::mt19937& rng) {
  const int64_t H = p.H, N = p.N, D = p.D, A = p.A, e = p.elem_bytes;
  std::vector<int32_t> pos(H * A);
  std::vector<uint8_t> ak(H * A * D * e), av(H * A * D * e);
  std::vector<int32_t> idx(2 * H * N);
  std::vector<uint16_t> g16(2 * H * N), sc(2 * H * N * (D / 32)), ze(2 * H * N * (D / 32));
  std::vector<uint8_t> flag(2 * H * N), codes(2 * H * N * D);
  for (int64_t h = 0; h < H; ++h)
    for (int64_t a = 0; a < A; ++a) pos[h * A + a] = (int32_t)(N - A + a);
  for (auto& x : ak) x = (uint8_t)rng();
  for (auto& x : av) x = (uint8_t)rng();
  for (int64_t i = 0; i < 2 * H * N; ++i) {
    idx[i] = (int32_t)(rng() % A);
    g16[i] = (uint16_t)rng();
  }
  for (auto& x : codes) x = (uint8_t)(rng() & 3);
  for (auto& x : sc) x = (uint16_t)rng();
  for (auto& x : ze) x = (uint16_t)rng();
  const bool hlm = p.params.codec == ANCHORKV_CODEC_HADAMARD_LM;
  if (hlm)
    for (int64_t i = 0; i < 2 * H * N; ++i) {
      for (int g = 1; g < D / 32; ++g) sc[i * (D / 32) + g] = 0;
      for (int g = 0; g < D / 32; ++g) ze[i * (D / 32) + g] = 0;
    }
  // flag the first eligible items (non-anchor tokens: t < N - A)
  int64_t left[2] = {p.joint ? (int64_t)p.R_total : p.R_K, p.joint ? 0 : (int64_t)p.R_V};
  for (int s = 0; s < 2; ++s)
    for (int64_t h = 0; h < H; ++h)
      for (int64_t t = 0; t < N - A; ++t) {
        int64_t& l = p.joint ? left[0] : left[s];
        if (l > 0) { flag[(s * H + h) * N + t] = 1; --l; }
      }
  anchorkv_unit_arrays in{pos.data(), ak.data(), av.data(), idx.data(), g16.data(), flag.data(), codes.data(),
                          sc.data(), ze.data()};
  std::vector<uint8_t> unit(p.unit_bytes);
  CHECK(anchorkv_unit_pack_host(&p, &in, unit.data()) == 0);
  std::vector<int32_t> pos2(H * A), idx2(2 * H * N);
  std::vector<uint8_t> ak2(ak.size()), av2(av.size()), flag2(flag.size()), codes2(codes.size());
  std::vector<uint16_t> g2(g16.size()), sc2(sc.size()), ze2(ze.size());
  anchorkv_unit_arrays out{pos2.data(), ak2.data(), av2.data(), idx2.data(), g2.data(), flag2.data(), codes2.data(),
                           sc2.data(), ze2.data()};
  CHECK(anchorkv_unit_unpack_host(&p, unit.data(), &out) == 0);
  CHECK(pos == pos2 && ak == ak2 && av == av2 && idx == idx2 && g16 == g2 && flag == flag2);
  for (int64_t i = 0; i < 2 * H * N; ++i)
    if (flag[i]) {
      CHECK(std::memcmp(&codes[i * D], &codes2[i * D], D) == 0);
      CHECK(std::memcmp(&sc[i * (D / 32)], &sc2[i * (D / 32)], 2 * (D / 32)) == 0);
    }
  // the header rebuilds the plan; a corrupted one is refused, not read past
  anchorkv_plan_info q;
  CHECK(anchorkv_plan_from_header(unit.data(), p.units, &q) == 0);
  CHECK(q.unit_bytes == p.unit_bytes && q.R_K == p.R_K && q.R_total == p.R_total && q.params.codec == p.params.codec);
  anchorkv_layout lay;
  CHECK(anchorkv_cache_layout(unit.data(), &lay) == 0 && lay.unit_bytes == p.unit_bytes);
  size_t wsb = 0;
  CHECK(anchorkv_decode_workspace_bytes(unit.data(), p.units, &wsb) == 0 && (int64_t)wsb == p.decode_workspace_bytes);
  for (int k = 0; k < 64; ++k) {
    std::vector<uint8_t> bad(unit.begin(), unit.begin() + 256);
    bad[rng() % 256] ^= (uint8_t)(1u << (rng() % 8));
    anchorkv_plan_info r;
    (void)anchorkv_plan_from_header(bad.data(), 1, &r);   // any return code, no invalid access
  }
  // an unpack whose flags disagree with the plan fails cleanly
  unit[p.off_words + 2] ^= 0x80;
  (void)anchorkv_unit_unpack_host(&p, unit.data(), &out);
}

int main() {
  std::mt19937 rng(12345);
  int planned = 0;
  for (int it = 0; it < 400; ++it) {
    anchorkv_dims d{1 + (int)(rng() % 2), 1 + (int)(rng() % 4), 1 + (int)(rng() % 8), 64 + (int)(rng() % 3000),
                    128, 1 + (int)(rng() % 32), 1 + (int)(rng() % 2)};
    anchorkv_params q;
    anchorkv_params_default(&q, 0.02f + 0.5f * (float)(rng() % 100) / 100.0f, 1 + (int)(rng() % 64));
    q.anchor_div = 1 + (int)(rng() % 200);
    q.rho = (double)(rng() % 11) / 10.0;
    q.pool = 1 + 2 * (int)(rng() % 8);
    q.pool_kv_jointly = (int)(rng() % 2);
    q.codec = (int)(rng() % 2);
    if (it % 17 == 0) q.pool = 4;            // invalid
    if (it % 19 == 0) q.codec = 7;           // invalid
    if (it % 23 == 0) d.head_dim = 64;       // invalid
    if (it % 29 == 0) d.n_obs = d.n_tokens + 1;
    anchorkv_plan_info p;
    const int rc = anchorkv_plan(&d, &q, &p);
    if (rc != 0) continue;
    ++planned;
    CHECK(p.unit_bytes <= p.unit_stride && p.cache_bytes == p.unit_stride * p.units);
    CHECK(p.used_bytes_k <= p.budget_bytes_per_side + 1 && p.R_K >= 0 && p.A >= p.window);
    if ((int64_t)p.H * p.N <= 4 * 3100) roundtrip(p, rng);
  }
  CHECK(anchorkv_plan(nullptr, nullptr, nullptr) != 0);
  CHECK(anchorkv_plan_from_header(nullptr, 1, nullptr) != 0);
  std::printf("planned %d shapes, %d failures\n", planned, failures);
  return failures == 0 && planned > 50 ? 0 : 1;
}
