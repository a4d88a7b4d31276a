// validate_main.cpp -- drives every argument check of the C ABI (fa_api.cpp) on the host, for the
// AddressSanitizer / UndefinedBehaviorSanitizer build of tests/test_abi_sanitizers.py.
//
// Pointers are fake device addresses: validation must decide from their values alone and never
// dereference them.  Every rejected call must return its status without reaching a launcher;
// every accepted call must reach the right launcher with the arguments it was given.  Extreme
// sizes (INT_MAX, products past 2^31 and 2^63) exercise the overflow checks, where the sanitizer
// would flag signed overflow.  Exits 0 when every check holds, 1 otherwise.
#include <climits>
#include <cmath>
#include <cstdio>
#include <cstring>

#include "fa.h"
#include "stub_launch.h"

namespace {

int failures = 0;

void expect(const char* what, fa_status got, fa_status want, const char* launcher) {
  const bool reached = stub::last.what != nullptr;
  bool ok = got == want;
  if (want == FA_OK)
    ok = ok && reached && std::strcmp(stub::last.what, launcher) == 0;
  else
    ok = ok && !reached;
  if (!ok) {
    std::printf("FAIL %s: status %d (want %d), launcher %s\n", what, (int)got, (int)want,
                reached ? stub::last.what : "none");
    ++failures;
  }
  stub::last = {};
}

#define CHECK(what, call, want, launcher) \
  do {                                    \
    stub::last = {};                      \
    expect(what, (call), want, launcher); \
  } while (0)

void* P(unsigned long a) { return reinterpret_cast<void*>(a); }
const int32_t* I(unsigned long a) { return reinterpret_cast<const int32_t*>(a); }
float* F(unsigned long a) { return reinterpret_cast<float*>(a); }

const unsigned long A = 0x10000;  // 16-byte aligned fake device addresses
const unsigned long Bp = 0x20000;
const unsigned long C = 0x30000;
const unsigned long Dp = 0x40000;
const unsigned long E = 0x50000;

void fwd() {
  auto call = [](const void* q, int B, int H, int Hkv, int N, int d, float scale, int dtype,
                 float* lse, const int32_t* sl) {
    return fa_fwd(q, P(Bp), P(C), P(Dp), lse, B, H, Hkv, N, d, scale, 0, sl, dtype, nullptr);
  };
  CHECK("fwd ok bf16", call(P(A), 1, 8, 8, 16384, 128, 0.088f, FA_BF16, F(E), nullptr), FA_OK,
        "fwd_bf16");
  CHECK("fwd ok f32", call(P(A), 1, 1, 1, 256, 64, 0.125f, FA_F32, F(E), I(E + 4)), FA_OK,
        "fwd_f32");
  CHECK("fwd null q", call(nullptr, 1, 8, 8, 64, 128, 0.1f, FA_BF16, F(E), nullptr),
        FA_ERR_INVALID_ARG, "");
  CHECK("fwd null lse", call(P(A), 1, 8, 8, 64, 128, 0.1f, FA_BF16, nullptr, nullptr),
        FA_ERR_INVALID_ARG, "");
  CHECK("fwd B=0", call(P(A), 0, 8, 8, 64, 128, 0.1f, FA_BF16, F(E), nullptr), FA_ERR_INVALID_ARG, "");
  CHECK("fwd N<0", call(P(A), 1, 8, 8, -5, 128, 0.1f, FA_BF16, F(E), nullptr), FA_ERR_INVALID_ARG, "");
  CHECK("fwd H%Hkv", call(P(A), 1, 8, 3, 64, 128, 0.1f, FA_BF16, F(E), nullptr),
        FA_ERR_INVALID_ARG, "");
  CHECK("fwd scale nan", call(P(A), 1, 8, 8, 64, 128, NAN, FA_BF16, F(E), nullptr),
        FA_ERR_INVALID_ARG, "");
  CHECK("fwd scale inf", call(P(A), 1, 8, 8, 64, 128, INFINITY, FA_BF16, F(E), nullptr),
        FA_ERR_INVALID_ARG, "");
  CHECK("fwd scale <0", call(P(A), 1, 8, 8, 64, 128, -1.f, FA_BF16, F(E), nullptr),
        FA_ERR_INVALID_ARG, "");
  CHECK("fwd misaligned q", call(P(A + 8), 1, 8, 8, 64, 128, 0.1f, FA_BF16, F(E), nullptr),
        FA_ERR_INVALID_ARG, "");
  CHECK("fwd misaligned lse", call(P(A), 1, 8, 8, 64, 128, 0.1f, FA_BF16, F(E + 2), nullptr),
        FA_ERR_INVALID_ARG, "");
  CHECK("fwd misaligned seq_lens", call(P(A), 1, 8, 8, 64, 128, 0.1f, FA_BF16, F(E), I(E + 1)),
        FA_ERR_INVALID_ARG, "");
  CHECK("fwd dtype", call(P(A), 1, 8, 8, 64, 128, 0.1f, 7, F(E), nullptr), FA_ERR_UNSUPPORTED, "");
  CHECK("fwd d=96", call(P(A), 1, 8, 8, 64, 96, 0.1f, FA_BF16, F(E), nullptr), FA_ERR_UNSUPPORTED, "");
  CHECK("fwd grid overflow", call(P(A), INT_MAX, INT_MAX, 1, INT_MAX, 128, 0.1f, FA_BF16, F(E), nullptr),
        FA_ERR_UNSUPPORTED, "");
  CHECK("fwd N past 2^30", call(P(A), 1, 1, 1, INT_MAX, 64, 0.1f, FA_BF16, F(E), nullptr),
        FA_ERR_UNSUPPORTED, "");
  CHECK("fwd N at the cap", call(P(A), 1, 1, 1, INT_MAX / 2, 64, 0.1f, FA_BF16, F(E), nullptr), FA_OK,
        "fwd_bf16");
}

void fp8() {
  auto call = [](float qs, int N, int d, const void* o) {
    return fa_fwd_fp8(P(A), P(Bp), P(C), qs, 1.f, 1.f, const_cast<void*>(o), F(E), 1, 8, 2, N, d,
                      0.1f, 1, nullptr, nullptr);
  };
  CHECK("fp8 ok", call(0.01f, 4096, 128, P(Dp)), FA_OK, "fwd_fp8");
  CHECK("fp8 descale nan", call(NAN, 4096, 128, P(Dp)), FA_ERR_INVALID_ARG, "");
  CHECK("fp8 descale <0", call(-1.f, 4096, 128, P(Dp)), FA_ERR_INVALID_ARG, "");
  CHECK("fp8 null o", call(1.f, 4096, 128, nullptr), FA_ERR_INVALID_ARG, "");
  CHECK("fp8 misaligned o", call(1.f, 4096, 128, P(Dp + 4)), FA_ERR_INVALID_ARG, "");
  CHECK("fp8 d=32", call(1.f, 4096, 32, P(Dp)), FA_ERR_UNSUPPORTED, "");
  CHECK("fp8 N=0", call(1.f, 0, 128, P(Dp)), FA_ERR_INVALID_ARG, "");
  CHECK("fp8 N=INT_MAX", call(1.f, INT_MAX, 128, P(Dp)), FA_ERR_UNSUPPORTED, "");
}

void bwd() {
  const size_t need = fa_bwd_workspace_bytes(2, 8, 1000);
  auto call = [](int B, int N, int dtype, const void* ws, size_t wsb) {
    return fa_bwd(P(A), P(Bp), P(C), P(Dp), F(E), P(A), P(Bp), P(C), P(Dp), B, 8, 2, N, 128, 0.1f,
                  0, nullptr, dtype, const_cast<void*>(ws), wsb, nullptr);
  };
  CHECK("bwd ok", call(2, 1000, FA_BF16, P(E), need), FA_OK, "bwd_bf16");
  CHECK("bwd workspace short", call(2, 1000, FA_BF16, P(E), need - 1), FA_ERR_INVALID_ARG, "");
  CHECK("bwd workspace null", call(2, 1000, FA_BF16, nullptr, need), FA_ERR_INVALID_ARG, "");
  CHECK("bwd workspace misaligned", call(2, 1000, FA_BF16, P(E + 8), need), FA_ERR_INVALID_ARG, "");
  CHECK("bwd f32", call(2, 1000, FA_F32, P(E), need), FA_ERR_UNSUPPORTED, "");
  CHECK("bwd rows overflow", call(INT_MAX, INT_MAX, FA_BF16, P(E), (size_t)-1), FA_ERR_UNSUPPORTED, "");
  CHECK("bwd N=INT_MAX", call(1, INT_MAX, FA_BF16, P(E), (size_t)-1), FA_ERR_UNSUPPORTED, "");
  if (fa_bwd_workspace_bytes(0, 8, 10) != 0 || fa_bwd_workspace_bytes(1, 1, -3) != 0) {
    std::printf("FAIL bwd workspace size of empty shapes\n");
    ++failures;
  }
}

void unfused() {
  const size_t need = fa_fwd_unfused_workspace_bytes(1, 8, 4096);
  auto call = [](int N, size_t wsb) {
    return fa_fwd_unfused(P(A), P(Bp), P(C), P(Dp), F(E), 1, 8, 8, N, 128, 0.1f, 0, P(E), wsb,
                          nullptr);
  };
  CHECK("unfused ok", call(4096, need), FA_OK, "fwd_unfused");
  CHECK("unfused short", call(4096, need - 16), FA_ERR_INVALID_ARG, "");
  CHECK("unfused N%8", call(4100, (size_t)-1), FA_ERR_UNSUPPORTED, "");
  CHECK("unfused rows overflow", call(INT_MAX - 7, (size_t)-1), FA_ERR_UNSUPPORTED, "");
}

void prefill() {
  const size_t need = fa_paged_prefill_workspace_bytes(16, 1024, 32, 8, 128, 2048);
  auto call = [](int S, int max_q, int Hq, int Hkv, int bs, int mb, int nb, const int32_t* ql,
                 const void* ws = P(E), size_t wsb = (size_t)-1) {
    return fa_paged_prefill(P(A), P(Bp), P(C), I(Dp), I(Dp + 4), ql, P(E), F(E), S, max_q, Hq, Hkv,
                            128, bs, mb, nb, 0.1f, const_cast<void*>(ws), wsb, nullptr);
  };
  CHECK("prefill ok", call(16, 1024, 32, 8, 16, 2048, 4096, I(Dp + 8), P(E), need), FA_OK,
        "paged_prefill");
  CHECK("prefill short workspace", call(16, 1024, 32, 8, 16, 2048, 4096, I(Dp + 8), P(E), need - 1),
        FA_ERR_INVALID_ARG, "");
  CHECK("prefill null workspace", call(16, 1024, 32, 8, 16, 2048, 4096, I(Dp + 8), nullptr),
        FA_ERR_INVALID_ARG, "");
  CHECK("prefill misaligned workspace", call(16, 1024, 32, 8, 16, 2048, 4096, I(Dp + 8), P(E + 8)),
        FA_ERR_INVALID_ARG, "");
  CHECK("prefill null q_lens", call(16, 1024, 32, 8, 16, 2048, 4096, nullptr), FA_ERR_INVALID_ARG, "");
  CHECK("prefill misaligned q_lens", call(16, 1024, 32, 8, 16, 2048, 4096, I(Dp + 2)),
        FA_ERR_INVALID_ARG, "");
  CHECK("prefill num_blocks 0", call(16, 1024, 32, 8, 16, 2048, 0, I(Dp + 8)), FA_ERR_INVALID_ARG, "");
  CHECK("prefill block 32", call(16, 1024, 32, 8, 32, 2048, 4096, I(Dp + 8)), FA_ERR_UNSUPPORTED, "");
  CHECK("prefill tokens overflow", call(16, 1024, 32, 8, 16, INT_MAX, 4096, I(Dp + 8)),
        FA_ERR_UNSUPPORTED, "");
  CHECK("prefill grid overflow", call(INT_MAX, INT_MAX, INT_MAX, 1, 16, 64, 4096, I(Dp + 8)),
        FA_ERR_UNSUPPORTED, "");
  CHECK("prefill items overflow", call(1 << 16, 1 << 16, 64, 64, 16, 64, 4096, I(Dp + 8)),
        FA_ERR_UNSUPPORTED, "");
  CHECK("prefill max_q=INT_MAX", call(1, INT_MAX, 1, 1, 16, 64, 4096, I(Dp + 8)),
        FA_ERR_UNSUPPORTED, "");
  if (fa_paged_prefill_workspace_bytes(0, 1024, 32, 8, 128, 2048) != 0 ||
      fa_paged_prefill_workspace_bytes(16, 1024, 32, 5, 128, 2048) != 0) {
    std::printf("FAIL prefill workspace size of invalid shapes\n");
    ++failures;
  }
}

void decode() {
  const size_t need = fa_paged_decode_workspace_bytes(64, 32, 128, 2048, 16);
  auto call = [](int S, int Hq, int Hkv, int bs, int mb, int nb, const void* ws, size_t wsb) {
    return fa_paged_decode(P(A), P(Bp), P(C), I(Dp), I(Dp + 4), P(E), F(E), S, Hq, Hkv, 128, bs, mb,
                           nb, 0.1f, const_cast<void*>(ws), wsb, nullptr);
  };
  CHECK("decode ok", call(64, 32, 8, 16, 2048, 4096, P(E), need), FA_OK, "paged_decode");
  CHECK("decode short workspace", call(64, 32, 8, 16, 2048, 4096, P(E), need - 4),
        FA_ERR_INVALID_ARG, "");
  CHECK("decode group 32", call(64, 64, 2, 16, 2048, 4096, P(E), (size_t)-1), FA_ERR_UNSUPPORTED, "");
  CHECK("decode block 8", call(64, 32, 8, 8, 2048, 4096, P(E), (size_t)-1), FA_ERR_UNSUPPORTED, "");
  CHECK("decode num_blocks <0", call(64, 32, 8, 16, 2048, -1, P(E), (size_t)-1),
        FA_ERR_INVALID_ARG, "");
  CHECK("decode tokens overflow", call(64, 32, 8, 16, INT_MAX, 4096, P(E), (size_t)-1),
        FA_ERR_UNSUPPORTED, "");
  CHECK("decode grid overflow", call(INT_MAX, 32, 8, 16, 2048, 4096, P(E), (size_t)-1),
        FA_ERR_UNSUPPORTED, "");
  if (fa_paged_decode_workspace_bytes(0, 32, 128, 2048, 16) != 0) {
    std::printf("FAIL decode workspace size of an empty batch\n");
    ++failures;
  }
  // Extreme sizes must not overflow inside the size arithmetic (the sanitizer checks the signed
  // intermediate products).
  (void)fa_paged_decode_workspace_bytes(INT_MAX, INT_MAX, 128, INT_MAX, 16);
  (void)fa_bwd_workspace_bytes(INT_MAX, INT_MAX, INT_MAX);
  (void)fa_fwd_unfused_workspace_bytes(INT_MAX, INT_MAX, 65536);
}

void decode_noalloc() {
  auto call = [](int S, int Hq, int Hkv, int mb, const void* q) {
    return fa_paged_decode_noalloc(q, P(Bp), P(C), I(Dp), I(Dp + 4), P(E), F(E), S, Hq, Hkv, 128,
                                   16, mb, 4096, 0.1f, nullptr);
  };
  CHECK("noalloc ok", call(64, 32, 8, 2048, P(A)), FA_OK, "paged_decode_noalloc");
  CHECK("noalloc too large", call(64, 32, 8, 4096, P(A)), FA_ERR_TOO_LARGE, "");
  CHECK("noalloc null q", call(64, 32, 8, 2048, nullptr), FA_ERR_INVALID_ARG, "");
  CHECK("noalloc grid overflow", call(INT_MAX, 32, 8, 2048, P(A)), FA_ERR_UNSUPPORTED, "");
}

}  // namespace

int main() {
  fwd();
  fp8();
  bwd();
  unfused();
  prefill();
  decode();
  decode_noalloc();
  for (int s = 0; s <= 4; ++s)
    if (fa_status_str((fa_status)s) == nullptr) ++failures;
  std::printf("%s (%d failures)\n", failures ? "FAILED" : "all validation checks hold", failures);
  return failures ? 1 : 0;
}
