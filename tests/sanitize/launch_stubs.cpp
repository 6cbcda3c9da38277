// Host-only stand-ins for the kernel launchers of libdsv4attn, for building
// the C ABI (api.cpp) and the planners (plan.cpp) with the host sanitizers:
// every launcher returns success without touching memory, so argument
// checks, size queries and launch plans run exactly as in the library while
// no kernel runs.  Test infrastructure only; never linked into the library.
#include "dsv4_internal.h"

namespace dsv4 {

hipError_t launch_csa_compress(const CompressArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_hca_compress(const CompressArgs&, hipStream_t) { return hipSuccess; }
bool compress_fused_ok(const CompressArgs*, const CompressArgs*, const CompressArgs*) { return false; }
hipError_t launch_compress_fused(const CompressArgs*, const CompressArgs*, const CompressArgs*, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_indexer(const IndexerArgs&, const int64_t*, hipStream_t) { return hipSuccess; }
hipError_t launch_indexer_topk(const IndexerArgs& a, const int64_t*, int k, int32_t*, void*, hipStream_t) {
  // the plan the real launcher builds for each slice
  for (int64_t b0 = 0; b0 < a.B; b0 += MAXB) {
    IndexerArgs s = a;
    s.B = a.B - b0 < MAXB ? a.B - b0 : MAXB;
    (void)idxtopk_make_plan(s, k);
  }
  return hipSuccess;
}
hipError_t launch_topk(const float*, int64_t, int64_t, int64_t, int, const int64_t*, int, int32_t*, void*,
                       const TopkPlan&, hipStream_t) {
  return hipSuccess;
}
hipError_t topk_scratch_ptr(void** ptr) {
  *ptr = reinterpret_cast<void*>(static_cast<uintptr_t>(0x10000));
  return hipSuccess;
}
hipError_t launch_attn(const AttnArgs&, const int64_t*, const int64_t*, const AttnLaunchPlan&, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_q_prep(const QPrepArgs&, const int64_t*, hipStream_t) { return hipSuccess; }
hipError_t launch_kv_prep(const KvPrepArgs&, const int64_t*, hipStream_t) { return hipSuccess; }
hipError_t launch_stream_reset(void*, int64_t, int, int, int, hipStream_t) { return hipSuccess; }
hipError_t launch_stream(const StreamArgs&, const int64_t*, const int64_t*, hipStream_t) { return hipSuccess; }
hipError_t launch_gemm(const GemmArgs&, hipStream_t) { return hipSuccess; }

}  // namespace dsv4
