// Host stand-ins for the device code, so the C ABI can be driven on a machine without a
// GPU (tests/test_host_sanitizers.py); the drive reaches none of them.
#include <cstdlib>
#include "../../memory_bounded_streaming_amd/csrc/kernels.hpp"
#include "../../memory_bounded_streaming_amd/csrc/engine.hpp"
namespace cqsa {
int attn_query_tile(cqsa_dtype dtype) { return dtype == CQSA_BF16 ? kAttnQueryTileBf16 : kAttnQueryTileF32; }
hipError_t launch_attn(const AttnLaunch&, hipStream_t) { std::abort(); }
hipError_t launch_merge(const MergeLaunch&, hipStream_t) { std::abort(); }
int bwd_key_tile(cqsa_dtype) { return 128; }
int bwd_query_tile(cqsa_dtype) { return 128; }
hipError_t launch_accumulate(const AccLaunch&, hipStream_t) { std::abort(); }
hipError_t launch_bwd_prep(const PrepLaunch&, hipStream_t) { std::abort(); }
hipError_t launch_bwd_dkdv(const BwdLaunch&, hipStream_t) { std::abort(); }
hipError_t launch_bwd_dq(const BwdLaunch&, hipStream_t) { std::abort(); }
hipError_t launch_sum_slots(const SumLaunch&, hipStream_t) { std::abort(); }
cqsa_status forward_static(const Plan&, const void*, const void*, const void*, void*, float*, hipStream_t, std::string&) { std::abort(); }
int64_t static_scratch_capacity() { return int64_t(256) << 20; }
int64_t static_scratch_need(const Plan&) { return 0; }
}
