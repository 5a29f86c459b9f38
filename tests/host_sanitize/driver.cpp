// Drives every entry point of the C ABI (api.cpp, built with
// AddressSanitizer and UndefinedBehaviorSanitizer against stub launchers)
// through invalid arguments, the supported limits and geometries past the
// int32 limits, checking the status codes and that rejected calls launch
// nothing.  No device pointer is ever dereferenced on the host, so fake
// addresses stand in for them.  Exits non-zero on the first failed check; a
// sanitizer report aborts the process.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <initializer_list>

#include "../../include/moba.h"

extern long long g_launches;

namespace {

int g_checks = 0;
#define CHECK(cond)                                                          \
  do {                                                                       \
    ++g_checks;                                                              \
    if (!(cond)) {                                                           \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      std::exit(1);                                                          \
    }                                                                        \
  } while (0)

void* const FAKE = reinterpret_cast<void*>(uintptr_t{1} << 40);  // 256-byte aligned
const int32_t* const CU = static_cast<const int32_t*>(FAKE);

struct G {
  int S = 1, T = 1000, L = 1000, NB = 8, H = 2, d = 128, B = 128;
};

int pool(const G& g, int dtype = MOBA_BF16, void* k = FAKE, void* kbar = FAKE) {
  return moba_pool_keys(k, dtype, CU, CU, g.S, g.T, g.L, g.NB, g.H, g.d, g.B,
                        static_cast<float*>(kbar), static_cast<uint16_t*>(FAKE), nullptr);
}
int gate(const G& g, int topk, int dtype = MOBA_BF16, const void* kbar3 = FAKE) {
  return moba_gate_topk(FAKE, dtype, static_cast<const float*>(FAKE),
                        static_cast<const uint16_t*>(kbar3), CU, CU, g.S, g.T, g.L, g.NB, g.H,
                        g.d, g.B, topk, static_cast<int32_t*>(FAKE), nullptr);
}
int fwd(const G& g, int topk, int head_chunk, size_t ws_bytes, int dtype = MOBA_BF16,
        float scale = 0.1f, void* ws = FAKE) {
  return moba_attn_fwd(FAKE, FAKE, FAKE, dtype, CU, CU, g.S, g.T, g.L, g.NB, g.H, g.d, g.B, topk,
                       CU, scale, FAKE, MOBA_BF16, static_cast<float*>(FAKE), head_chunk, ws,
                       ws_bytes, nullptr);
}
size_t fwd_bytes(const G& g, int topk, int head_chunk, int dtype = MOBA_BF16) {
  return moba_attn_workspace_bytes(dtype, g.T, g.NB, g.H, g.d, g.B, topk, head_chunk);
}
int nblocks(long long T, int B) { return (int)((T + B - 1) / B); }

}  // namespace

int main() {
  CHECK(moba_api_version() == MOBA_API_VERSION);
  for (int s : {0, -1, -2, -3, -4, 7, -99}) CHECK(moba_status_str(s) != nullptr);

  G g;
  // pool and gate: invalid arguments launch nothing
  long long before = g_launches;
  CHECK(pool(g, MOBA_BF16, nullptr) == MOBA_ERR_INVALID_ARG);
  CHECK(pool(g, MOBA_BF16, FAKE, nullptr) == MOBA_ERR_INVALID_ARG);
  CHECK(pool(g, 7) == MOBA_ERR_INVALID_ARG);
  {
    G b = g;
    b.NB = 7;  // fewer blocks than ceil(T / B)
    CHECK(pool(b) == MOBA_ERR_INVALID_ARG);
    b = g;
    b.B = 96;
    CHECK(pool(b) == MOBA_ERR_UNSUPPORTED);
    b = g;
    b.d = 96;
    CHECK(pool(b) != MOBA_OK);
    b = g;
    b.L = 1001;
    CHECK(pool(b) == MOBA_ERR_INVALID_ARG);
  }
  CHECK(gate(g, 3, MOBA_BF16, nullptr) == MOBA_ERR_INVALID_ARG);
  CHECK(gate(g, 0) == MOBA_ERR_INVALID_ARG);
  CHECK(g_launches == before);
  CHECK(pool(g) == MOBA_OK);
  CHECK(gate(g, 3) == MOBA_OK);
  CHECK(gate(g, 3, MOBA_F32, nullptr) == MOBA_OK);  // fp32 queries read kbar only
  CHECK(g_launches > before);

  // forward: workspace sizes for every head pass, the reported size accepted,
  // half of it refused before any launch
  for (int H : {1, 3, 32}) {
    for (int topk : {1, 2, 12, 64}) {
      G f = g;
      f.H = H;
      f.T = 5000;
      f.L = 5000;
      f.NB = nblocks(5000, 128);
      size_t prev = 0;
      for (int hc = 1; hc <= H; ++hc) {
        const size_t need = fwd_bytes(f, topk, hc);
        CHECK(need > 0);
        CHECK(need >= prev);  // grows with the heads per pass
        prev = need;
        before = g_launches;
        CHECK(fwd(f, topk, hc, need / 2) == MOBA_ERR_WORKSPACE_TOO_SMALL);
        CHECK(g_launches == before);
        CHECK(fwd(f, topk, hc, need) == MOBA_OK);
        CHECK(g_launches > before);
      }
      CHECK(fwd_bytes(f, topk, 0) == fwd_bytes(f, topk, H));
      CHECK(fwd(f, topk, 0, fwd_bytes(f, topk, 0)) == MOBA_OK);
    }
  }
  // invalid forward arguments
  before = g_launches;
  CHECK(fwd(g, 3, 0, 1ull << 40, MOBA_BF16, 0.0f) == MOBA_ERR_INVALID_ARG);
  CHECK(fwd(g, 3, -1, 1ull << 40) == MOBA_ERR_INVALID_ARG);
  CHECK(fwd(g, 0, 0, 1ull << 40) == MOBA_ERR_INVALID_ARG);
  CHECK(fwd(g, 65, 0, 1ull << 40) != MOBA_OK);
  CHECK(fwd(g, 3, 0, 1ull << 40, MOBA_BF16, 0.1f, nullptr) == MOBA_ERR_INVALID_ARG);
  CHECK(fwd(g, 3, 0, 1ull << 40, MOBA_BF16, 0.1f, (char*)FAKE + 16) == MOBA_ERR_INVALID_ARG);
  CHECK(g_launches == before);
  // past the int32 limits of the lists: refused as unsupported in one pass,
  // accepted in passes of fewer heads
  {
    G big;
    big.T = 1 << 20;
    big.L = 1 << 20;
    big.B = 4096;
    big.NB = 256;
    big.H = 256;
    const int topk = 12;  // 2^20 * 256 * 11 entries > 2^31
    CHECK(fwd(big, topk, 0, ~size_t{0}) == MOBA_ERR_UNSUPPORTED);
    CHECK(fwd(big, topk, 32, fwd_bytes(big, topk, 32)) == MOBA_OK);
  }
  // the largest token counts the workspace arithmetic sees stay defined
  for (int topk : {2, 12, 64}) {
    G huge;
    huge.T = 2000000000 / topk;
    huge.L = huge.T;
    huge.B = 4096;
    huge.NB = nblocks(huge.T, 4096);
    huge.H = 128;
    for (int hc : {0, 1, 7, 128}) (void)fwd_bytes(huge, topk, hc);
  }
  // the fixed-workspace entry point: small layers fit, a head that needs
  // more than the array is refused before any launch
  before = g_launches;
  CHECK(moba_attn_fwd_static(FAKE, FAKE, FAKE, MOBA_BF16, CU, CU, g.S, g.T, g.L, g.NB, g.H, g.d,
                             g.B, 3, CU, 0.1f, FAKE, MOBA_BF16, static_cast<float*>(FAKE),
                             nullptr) == MOBA_OK);
  CHECK(g_launches > before);
  {
    G big;
    big.T = 1 << 20;
    big.L = 1 << 20;
    big.B = 4096;
    big.NB = 256;
    big.H = 4;
    before = g_launches;
    CHECK(moba_attn_fwd_static(FAKE, FAKE, FAKE, MOBA_BF16, CU, CU, big.S, big.T, big.L, big.NB,
                               big.H, big.d, big.B, 12, CU, 0.1f, FAKE, MOBA_BF16,
                               static_cast<float*>(FAKE), nullptr) ==
          MOBA_ERR_WORKSPACE_TOO_SMALL);
    CHECK(g_launches == before);
  }
  // dense
  {
    const size_t need = moba_dense_workspace_bytes(MOBA_BF16, g.T, g.NB, g.H, g.d, g.B);
    CHECK(need > 0);
    CHECK(moba_dense_causal_fwd(FAKE, FAKE, FAKE, MOBA_BF16, CU, CU, g.S, g.T, g.L, g.NB, g.H,
                                g.d, g.B, 0.1f, FAKE, MOBA_F32, static_cast<float*>(FAKE), FAKE,
                                need / 2, nullptr) == MOBA_ERR_WORKSPACE_TOO_SMALL);
    CHECK(moba_dense_causal_fwd(FAKE, FAKE, FAKE, MOBA_BF16, CU, CU, g.S, g.T, g.L, g.NB, g.H,
                                g.d, g.B, 0.1f, FAKE, MOBA_F32, static_cast<float*>(FAKE), FAKE,
                                need, nullptr) == MOBA_OK);
  }
  // backward
  for (int topk : {1, 3, 12}) {
    const size_t need = moba_attn_bwd_workspace_bytes(MOBA_BF16, g.T, g.NB, g.H, g.d, g.B, topk);
    CHECK(need > 0);
    auto bwd = [&](size_t bytes) {
      return moba_attn_bwd(FAKE, FAKE, FAKE, FAKE, MOBA_F32, FAKE, static_cast<const float*>(FAKE),
                           MOBA_BF16, CU, CU, g.S, g.T, g.L, g.NB, g.H, g.d, g.B, topk, CU, 0.1f,
                           static_cast<float*>(FAKE), static_cast<float*>(FAKE),
                           static_cast<float*>(FAKE), FAKE, bytes, nullptr);
    };
    before = g_launches;
    CHECK(bwd(need / 2) == MOBA_ERR_WORKSPACE_TOO_SMALL);
    CHECK(g_launches == before);
    CHECK(bwd(need) == MOBA_OK);
  }
  // min/max gate and static routing
  CHECK(moba_pool_minmax(FAKE, MOBA_BF16, CU, CU, g.S, g.T, g.L, g.NB, g.H, g.d, g.B,
                         static_cast<float*>(FAKE), nullptr) == MOBA_OK);
  CHECK(moba_gate_topk_minmax(FAKE, MOBA_F32, static_cast<const float*>(FAKE), CU, CU, g.S, g.T,
                              g.L, g.NB, g.H, g.d, g.B, 3, static_cast<int32_t*>(FAKE),
                              nullptr) == MOBA_ERR_UNSUPPORTED);
  CHECK(moba_gate_topk_minmax(FAKE, MOBA_BF16, static_cast<const float*>(FAKE), CU, CU, g.S, g.T,
                              g.L, g.NB, g.H, g.d, g.B, 3, static_cast<int32_t*>(FAKE),
                              nullptr) == MOBA_OK);
  for (int sink : {-1, 0, 1, 5}) {
    const int st = moba_static_select(CU, CU, g.S, g.T, g.L, g.NB, g.H, g.B, 3, sink,
                                      static_cast<int32_t*>(FAKE), nullptr);
    CHECK(sink < 0 ? st == MOBA_ERR_INVALID_ARG : st == MOBA_OK);
  }
  // empty batches launch nothing and succeed
  {
    G e;
    e.T = 0;
    e.L = 0;
    e.NB = 0;
    before = g_launches;
    CHECK(pool(e) == MOBA_OK);
    CHECK(gate(e, 3) == MOBA_OK);
    CHECK(fwd(e, 3, 0, 1ull << 20) == MOBA_OK);
    CHECK(g_launches == before);
  }
  // profiler bookkeeping (host only: nothing attached, so nothing recorded)
  moba_profiler* p = nullptr;
  CHECK(moba_profiler_create(&p) == MOBA_OK && p != nullptr);
  char names[64];
  CHECK(moba_profiler_names(p, names, sizeof names) == MOBA_OK);
  int n = -1;
  double ms = -1.0;
  CHECK(moba_profiler_read(p, "pool_keys", &n, &ms) == MOBA_OK && n == 0);
  moba_profiler_destroy(p);

  std::printf("host sanitizer checks passed: %d\n", g_checks);
  return 0;
}
