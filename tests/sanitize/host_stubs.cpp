// Stand-ins for the device launches of libpbq, for a host-only build of the
// allocator and the C ABI (pool.cpp, capi.cpp) under AddressSanitizer and
// UndefinedBehaviorSanitizer (tests/test_sanitized_host.py).  The tests run
// on that build reach a launch only through an argument the C ABI accepted,
// which must then fail visibly: every stand-in returns an error.  The one
// host-side helper with a result, stream_read_groups, computes what
// stream_read.hip does (four waves per work group).

#include "pbq_internal.h"

namespace pbq {

hipError_t scratch_address(void** out) {
    *out = nullptr;
    return hipErrorNotSupported;
}
hipError_t launch_quantize_store(const QuantStoreArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_stream_read(const StreamReadArgs&, hipStream_t) { return hipErrorNotSupported; }
int64_t stream_read_groups(int64_t n_tiles, int64_t tiles_per_wave) {
    const int64_t waves = (n_tiles + tiles_per_wave - 1) / tiles_per_wave;
    return (waves + 3) / 4;
}
hipError_t launch_paged_attn(const AttnArgs&, hipStream_t) { return hipErrorNotSupported; }
bool split_store_fused(const AttnArgs&) { return false; }
hipError_t launch_copy_blocks(const CopyArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_swap_blocks(const SwapArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace pbq
