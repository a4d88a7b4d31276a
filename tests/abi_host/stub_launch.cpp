// stub_launch.cpp -- host-only stand-ins for the kernel launchers, for the sanitizer build of
// the C-ABI validation (tests/test_abi_sanitizers.py).  Each records that it was reached and the
// arguments it was given, and reports success; no device code and no HIP runtime are involved.
#include "stub_launch.h"

namespace stub {
Last last;
}

namespace fa {

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t) {
  stub::last = {"fwd_bf16", a.B, a.H, a.Hkv, a.N, a.d, 0};
  return hipSuccess;
}
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t) {
  stub::last = {"fwd_f32", a.B, a.H, a.Hkv, a.N, a.d, 0};
  return hipSuccess;
}
hipError_t launch_fwd_fp8(const Fp8FwdArgs& a, hipStream_t) {
  stub::last = {"fwd_fp8", a.B, a.H, a.Hkv, a.N, a.d, 0};
  return hipSuccess;
}
hipError_t launch_fwd_unfused(const UnfusedArgs& a, hipStream_t) {
  stub::last = {"fwd_unfused", a.B, a.H, a.Hkv, a.N, a.d, 0};
  return hipSuccess;
}
hipError_t launch_paged_prefill(const PagedPrefillArgs& a, hipStream_t) {
  stub::last = {"paged_prefill", a.S, a.Hq, a.Hkv, a.max_q, a.d, a.num_blocks};
  return hipSuccess;
}
hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t) {
  stub::last = {"bwd_bf16", a.B, a.H, a.Hkv, a.N, a.d, 0};
  return hipSuccess;
}
hipError_t launch_paged_decode(const DecodeArgs& a, hipStream_t) {
  stub::last = {"paged_decode", a.S, a.Hq, a.Hkv, a.max_blocks, a.d, a.num_blocks};
  return hipSuccess;
}

hipError_t launch_paged_decode_noalloc(DecodeArgs a, hipStream_t) {
  stub::last = {"paged_decode_noalloc", a.S, a.Hq, a.Hkv, a.max_blocks, a.d, a.num_blocks};
  return hipSuccess;
}

}  // namespace fa
