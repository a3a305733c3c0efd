// Test-support stubs (not part of the library): the launchers that the C ABI
// layer (exact_attention_74_amd/csrc/api.hip) dispatches to, replaced by
// functions that launch nothing and report "no device".  Linked with a
// host-only AddressSanitizer build of api.hip, they let the CPU tests drive
// every validation path, valid arguments included, without a GPU.
#include <stddef.h>

#include "launch.h"  // the declarations these definitions must match

namespace exattn {

hipError_t launch_attn_fwd_bf16(const void*, const void*, const void*, void*, float*, int, int, int,
                                int, int, bool, float, hipStream_t, bool) {
  return hipErrorNoDevice;
}
hipError_t launch_attn_fwd_fp8(const void*, const void*, const void*, const float*, const float*,
                               const float*, void*, float*, int, int, int, int, int, bool, float,
                               hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_attn_bwd_bf16(const void*, const void*, const void*, const void*, const void*,
                                const float*, void*, void*, void*, float*, int, int, int, int, int,
                                bool, float, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_attn_bwd_bf16_noalloc(const void*, const void*, const void*, const void*,
                                        const void*, const float*, void*, void*, void*, int, int,
                                        int, int, int, bool, float, hipStream_t) {
  return hipErrorNoDevice;
}
size_t bwd_scratch_bytes() { return size_t(16) << 20; }
hipError_t launch_blockquant(const void*, void*, float*, const float*, int, int, int, int, int,
                             hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_rope_blockquant(const void*, void*, float*, const float*, const float*,
                                  const float*, bool, int, int, int, int, int, hipStream_t) {
  return hipErrorNoDevice;
}

}  // namespace exattn
