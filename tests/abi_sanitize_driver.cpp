// Host-only driver for the sanitizer build of the C-ABI validator (run by
// tests/test_abi_host.py): every call here fails validation or is a
// workspace query, so nothing reaches the GPU.  Built with AddressSanitizer
// and UndefinedBehaviorSanitizer on the host code of csrc/abi.hip; any
// out-of-bounds access, use of freed memory, signed overflow or misaligned
// access in the validation and planning code aborts the run.  Exit status is
// the number of calls whose status differed from the expected one.
#include <cmath>
#include <cstdio>
#include <cstring>

#include "lora_mi355x.h"

static int g_fail = 0;

static void expect(const char* what, lora_status got, lora_status want) {
  if (got != want) {
    std::printf("FAIL %s: status %d, expected %d (%s)\n", what, (int)got, (int)want, lora_last_error());
    ++g_fail;
  }
}

int main() {
  void* const F = reinterpret_cast<void*>(uintptr_t(1) << 20);      // aligned, never dereferenced
  void* const F2 = reinterpret_cast<void*>(uintptr_t(1) << 21);
  void* const F3 = reinterpret_cast<void*>(uintptr_t(3) << 20);
  void* const ODD = reinterpret_cast<void*>((uintptr_t(1) << 20) + 2);
  size_t f = 0, b = 0;

  if (lora_version() != LORA_MI355X_VERSION) ++g_fail;
  for (int s = 0; s < 9; ++s) {
    lora_status st;  // 8 is no status: a C caller may still pass it
    std::memcpy(&st, &s, sizeof st);
    if (lora_strerror(st) == nullptr) ++g_fail;
  }
  float cb[16];
  lora_nf4_codebook(cb);
  for (int i = 1; i < 16; ++i)
    if (!(cb[i] > cb[i - 1])) ++g_fail;

  // gated MLP: workspace queries over valid and invalid descriptors, large and empty
  lora_mlp_desc d{8192, 4096, 14336, 16, LORA_ACT_SWIGLU, LORA_BF16, nullptr};
  expect("mlp ws", lora_mlp_workspace_size(&d, &f, &b), LORA_OK);
  lora_mlp_desc big{65535, 64, 16384, 16, LORA_ACT_GEGLU_TANH, LORA_BF16_F32LORA, nullptr};
  expect("mlp ws max extent", lora_mlp_workspace_size(&big, &f, &b), LORA_OK);
  lora_mlp_desc over{65536, 64, 16384, 16, LORA_ACT_SWIGLU, LORA_BF16, nullptr};
  expect("mlp ws 2 GiB", lora_mlp_workspace_size(&over, &f, &b), LORA_ESHAPE);
  lora_mlp_desc huge{int64_t(1) << 40, 4096, 14336, 16, LORA_ACT_SWIGLU, LORA_BF16, nullptr};
  expect("mlp ws overflowing T", lora_mlp_workspace_size(&huge, &f, &b), LORA_ESHAPE);
  lora_mlp_desc t0{0, 256, 512, 8, LORA_ACT_SWIGLU, LORA_F32, nullptr};
  expect("mlp ws T=0", lora_mlp_workspace_size(&t0, &f, &b), LORA_OK);
  lora_mlp_desc bad = d;
  bad.r = 12;
  expect("mlp r % 8", lora_mlp_workspace_size(&bad, &f, &b), LORA_ESHAPE);
  bad = d;
  bad.act = 5;
  expect("mlp act", lora_mlp_workspace_size(&bad, &f, &b), LORA_EINVAL);
  bad = d;
  bad.dtype = -1;
  expect("mlp dtype", lora_mlp_workspace_size(&bad, &f, &b), LORA_EDTYPE);
  expect("mlp null desc", lora_mlp_workspace_size(nullptr, &f, &b), LORA_EINVAL);
  lora_plan plan{};
  plan.gemm[1].ksplit = 4;
  plan.gemm[0].group = 16;
  bad = d;
  bad.plan = &plan;
  expect("mlp ws split plan", lora_mlp_workspace_size(&bad, &f, &b), LORA_OK);
  plan.gemm[0].group = 5;
  expect("mlp bad group", lora_mlp_workspace_size(&bad, &f, &b), LORA_EINVAL);

  lora_mlp_desc sd{300, 512, 1088, 16, LORA_ACT_SWIGLU, LORA_BF16, nullptr};
  lora_mlp_workspace_size(&sd, &f, &b);
  lora_proj p{F, nullptr, F2, F3, 2.0f};
  lora_proj pn{nullptr, nullptr, F2, F3, 2.0f};
  lora_proj pnan{F, nullptr, F2, F3, NAN};
  lora_mlp_saved sv{F, F2, F3};
  lora_mlp_saved svn{F, nullptr, F3};
  lora_mlp_grads gr{F, F, F, F, F, F};
  expect("mlp fwd X null", lora_mlp_fwd(&sd, nullptr, &p, &p, &p, F2, &sv, F3, f, nullptr), LORA_EINVAL);
  expect("mlp fwd X odd", lora_mlp_fwd(&sd, ODD, &p, &p, &p, F2, &sv, F3, f, nullptr), LORA_EALIGN);
  expect("mlp fwd no W", lora_mlp_fwd(&sd, F, &pn, &p, &p, F2, &sv, F3, f, nullptr), LORA_EINVAL);
  expect("mlp fwd nan scale", lora_mlp_fwd(&sd, F, &p, &pnan, &p, F2, &sv, F3, f, nullptr), LORA_EINVAL);
  expect("mlp fwd saved null", lora_mlp_fwd(&sd, F, &p, &p, &p, F2, &svn, F3, f, nullptr), LORA_EINVAL);
  expect("mlp fwd Y aliases X", lora_mlp_fwd(&sd, F, &p, &p, &p, F, &sv, F3, f, nullptr), LORA_EUNSUPPORTED);
  expect("mlp fwd small ws", lora_mlp_fwd(&sd, F, &p, &p, &p, F2, &sv, F3, f - 1, nullptr), LORA_EWORKSPACE);
  expect("mlp bwd grads null", lora_mlp_bwd(&sd, F, F2, &sv, &p, &p, &p, F3, nullptr, F3, b, nullptr), LORA_EINVAL);
  expect("mlp bwd dX overlaps X",
         lora_mlp_bwd(&sd, F, F2, &sv, &p, &p, &p, static_cast<char*>(F2) + 64, &gr, F3, b, nullptr),
         LORA_EUNSUPPORTED);
  expect("mlp bwd small ws", lora_mlp_bwd(&sd, F, F2, &sv, &p, &p, &p, F3, &gr, F3, b - 1, nullptr), LORA_EWORKSPACE);
  lora_plan act_split{};
  act_split.gemm[0].ksplit = 2;
  lora_mlp_desc sp = sd;
  sp.plan = &act_split;
  lora_mlp_workspace_size(&sp, &f, &b);
  expect("mlp fwd split of the activation GEMM", lora_mlp_fwd(&sp, F, &p, &p, &p, F2, &sv, F3, f, nullptr),
         LORA_EINVAL);

  // NF4 base with the fp32 compute dtype; shape mismatch; numel rule
  lora_nf4 q{static_cast<const uint8_t*>(F), static_cast<const int8_t*>(F2), static_cast<const float*>(F3),
             static_cast<const float*>(F), 512, 1088};
  lora_proj pq{nullptr, &q, F2, F3, 2.0f};
  lora_mlp_desc s32 = sd;
  s32.dtype = LORA_F32;
  lora_mlp_workspace_size(&s32, &f, &b);
  expect("mlp nf4 fp32", lora_mlp_fwd(&s32, F, &pq, &pq, &p, F2, &sv, F3, f, nullptr), LORA_EUNSUPPORTED);
  lora_mlp_workspace_size(&sd, &f, &b);
  lora_proj pqt{nullptr, &q, F2, F3, 2.0f, F};
  expect("mlp nf4 with Wt", lora_mlp_fwd(&sd, F, &pqt, &pq, &p, F2, &sv, F3, f, nullptr), LORA_EINVAL);
  lora_proj podd{F, nullptr, F2, F3, 2.0f, ODD};
  expect("mlp Wt odd", lora_mlp_fwd(&sd, F, &podd, &p, &p, F2, &sv, F3, f, nullptr), LORA_EALIGN);
  lora_nf4 qs{q.codes, q.q8, q.s2, q.mu, 64, 64};
  expect("nf4 dequant numel", lora_nf4_dequant(&qs, F, LORA_BF16, nullptr), LORA_ESHAPE);
  expect("nf4 unpack null", lora_nf4_unpack_codes(&q, nullptr, nullptr), LORA_EINVAL);
  expect("nf4 quantize ws", lora_nf4_quantize_workspace_size(64, 200, &f), LORA_ESHAPE);
  expect("nf4 gemm ws trans", lora_nf4_gemm_workspace_size(64, 256, 768, 16, 2, &f), LORA_EINVAL);
  expect("nf4 gemm ws extent", lora_nf4_gemm_workspace_size(int64_t(1) << 20, 256, 1024, 16, 0, &f), LORA_ESHAPE);
  expect("nf4 gemm A without B", lora_nf4_gemm(64, 0, F, &q, F2, nullptr, 16, 1.0f, F3, F, 1 << 20, nullptr),
         LORA_EINVAL);

  // ReLU^2, Q/K/V and O
  lora_relu2_mlp_desc rd{300, 256, 768, 64, LORA_BF16, 0, nullptr};
  expect("relu2 ws", lora_relu2_mlp_workspace_size(&rd, &f, &b), LORA_OK);
  rd.reserved = 1;
  expect("relu2 reserved", lora_relu2_mlp_workspace_size(&rd, &f, &b), LORA_EINVAL);
  lora_qkv_desc qd{8192, 4096, 4096, 1024, 1024, 16, LORA_BF16, 0, nullptr};
  expect("qkv ws", lora_qkv_workspace_size(&qd, &f, &b), LORA_OK);
  qd.r = 24;
  expect("qkv 3r > 64", lora_qkv_workspace_size(&qd, &f, &b), LORA_ESHAPE);
  lora_o_desc od{64, 256, 768, 16, LORA_BF16, 0, nullptr};
  expect("o ws", lora_o_workspace_size(&od, &f, &b), LORA_OK);
  lora_plan two{};
  two.gemm[1].group = 4;
  od.plan = &two;
  expect("o second plan entry", lora_o_workspace_size(&od, &f, &b), LORA_EINVAL);
  od.plan = nullptr;
  expect("o fwd noalloc over the scratch", [&] {
    lora_o_desc ob{300000, 64, 64, 8, LORA_BF16, 0, nullptr};
    return lora_o_fwd_noalloc(&ob, F, &p, F2, F3, nullptr);
  }(), LORA_EWORKSPACE);
  expect("o bwd dA null", lora_o_bwd(&od, F, F2, F3, &p, F, nullptr, F, F3, b, nullptr), LORA_EINVAL);

  // tracing without any launch
  expect("trace begin", lora_trace_begin("gemm"), LORA_OK);
  lora_trace_entry te[4];
  int32_t n = -1;
  expect("trace end", lora_trace_end(te, 4, &n), LORA_OK);
  if (n != 0) ++g_fail;

  std::printf("%d unexpected statuses\n", g_fail);
  return g_fail;
}
