// Host stand-ins for the kernel launchers, linked into the sanitizer build of
// the ABI layer (abi.cpp + plan.cpp): each counts that it was reached and
// reports success. Nothing here touches a GPU; the real launchers live in the
// .hip sources.
#include "../../attention_rope_amd/csrc/kernels.h"

namespace attn {
static int g_launches = 0;
static unsigned char g_scratch_stub[256];

hipError_t launch_prope(const void*, void*, const int32_t*, int, int, int, int, int, double, bool,
                        hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_rope_k_lead(const void*, void*, int, int, int, int, int, int, double, bool,
                              hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_prefill_cache_fill(const void*, const void*, void*, void*, void*,
                                     const int64_t*, int64_t, int, int, int, int, int, int, int,
                                     double, bool, hipStream_t) {
  ++g_launches; return hipSuccess;
}
hipError_t launch_prefill_mfma(const PrefillArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_prefill_mfma1w(const PrefillArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_prefill_mfma2g(const PrefillArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_prefill_general(const PrefillArgs&, bool, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_decode_merge(const DecodeArgs&, const SplitPlan&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_decode(const DecodeArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_kv_quantize_int8(const void*, int8_t*, float*, int, int, int, hipStream_t) {
  ++g_launches; return hipSuccess;
}
hipError_t launch_decode_int8(const DecodeArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t decode_scratch(void** ptr) { *ptr = g_scratch_stub; return hipSuccess; }
}  // namespace attn

extern "C" int stub_launches(void) { return attn::g_launches; }
