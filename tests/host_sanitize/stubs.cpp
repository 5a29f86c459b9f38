// Host-only stand-ins for the kernel launchers of launch.h, for the
// sanitizer build of the C-ABI layer (api.cpp): every launcher records that
// it was called and returns success without touching any pointer, so the
// ABI's argument checks, workspace arithmetic and pass loops run under
// AddressSanitizer and UndefinedBehaviorSanitizer with no GPU.
#include "../../block_sparse_long_03_amd/csrc/launch.h"
#include "../../include/moba.h"

long long g_launches = 0;  // read by the driver

namespace {
hipError_t launched() {
  ++g_launches;
  return hipSuccess;
}
}  // namespace

namespace moba {

hipError_t launch_pool_keys(const void*, bool, const Geo&, float*, uint16_t*, hipStream_t) {
  return launched();
}
hipError_t launch_gate_topk(const void*, bool, const float*, const uint16_t*, const Geo&, int,
                            int32_t*, hipStream_t) {
  return launched();
}
hipError_t launch_pool_minmax(const void*, bool, const Geo&, float*, hipStream_t) {
  return launched();
}
hipError_t launch_gate_topk_minmax(const uint16_t*, const float*, const Geo&, int, int32_t*,
                                   hipStream_t) {
  return launched();
}
hipError_t launch_static_select(const Geo&, int, int, int32_t*, hipStream_t) { return launched(); }
hipError_t launch_bucket(const int32_t*, const Geo&, int, int, int32_t*, int32_t*, int32_t*,
                         int32_t*, int4*, long long, hipStream_t, bool, int, int32_t*) {
  return launched();
}
hipError_t launch_v_transpose(const void*, const Geo&, uint32_t*, uint16_t*, hipStream_t) {
  return launched();
}
hipError_t launch_attn_mfma_hist(const void*, const void*, const uint16_t*, const Geo&, int, float,
                                 const int32_t*, const int4*, long long, uint16_t*, float*,
                                 hipStream_t) {
  return launched();
}
hipError_t launch_attn_mfma_own(const void*, const void*, const uint16_t*, const Geo&, int, float,
                                uint16_t*, float*, int, const int32_t*, hipStream_t) {
  return launched();
}
hipError_t launch_attn_mfma_dense(const void*, const void*, const uint16_t*, const uint32_t*,
                                  const Geo&, float, void*, bool, float*, hipStream_t, int) {
  return launched();
}
hipError_t launch_attn_f32_hist(const float*, const float*, const float*, const Geo&, int, float,
                                const int32_t*, const int32_t*, long long, float*, float*,
                                hipStream_t) {
  return launched();
}
hipError_t launch_attn_f32_own(const float*, const float*, const float*, const Geo&, int, float,
                               float*, float*, hipStream_t) {
  return launched();
}
hipError_t launch_attn_f32_dense(const float*, const float*, const float*, const Geo&, float,
                                 void*, bool, float*, hipStream_t) {
  return launched();
}
hipError_t launch_merge(const int32_t*, const Geo&, int, int, const void*, bool, const float*,
                        const uint32_t*, void*, bool, float*, hipStream_t) {
  return launched();
}
hipError_t launch_bwd_prep(const void*, bool, const uint16_t*, const float*, const Geo&, float*,
                           float*, float*, hipStream_t) {
  return launched();
}
hipError_t launch_bwd_kv(const uint16_t*, const uint16_t*, const uint16_t*, const uint16_t*,
                         const float*, const float*, const Geo&, int, float, const int32_t*,
                         const int32_t*, float*, float*, hipStream_t) {
  return launched();
}
hipError_t launch_bwd_q(const uint16_t*, const uint16_t*, const uint16_t*, const uint16_t*,
                        const float*, const float*, const Geo&, int, float, const int32_t*,
                        const int4*, long long, float*, hipStream_t) {
  return launched();
}
hipError_t static_workspace(void** ptr, size_t* bytes) {
  *ptr = reinterpret_cast<void*>(uintptr_t{1} << 40);  // never dereferenced
  *bytes = MOBA_STATIC_WORKSPACE_BYTES;
  return hipSuccess;
}
hipError_t launch_mfma_rate(int, int, int, float*, hipStream_t) { return launched(); }

}  // namespace moba
