// Host-only AddressSanitizer and UndefinedBehaviorSanitizer run of the C boundary's host
// side (include/gdn.h): every entry point with arguments it must reject, the workspace
// size queries and the status strings.  The kernel launchers are stubs that report a
// failed launch; none of the calls here gets as far as a launch, and the program exits
// 1 if one does.  Pointers are fake device addresses (never dereferenced on the host).
#include <stdio.h>
#include <string.h>

#include "gdn.h"
#include "gdn_kernels.h"

static int launches = 0;
namespace gdn {

#define STUB(sig) \
  hipError_t sig { \
    ++launches; \
    return hipErrorInvalidValue; \
  }
STUB(launch_bwd(const BwdParams &, int, int, int, bool, hipStream_t))
STUB(launch_fill_zero(float *, size_t, hipStream_t))
STUB(launch_sum_tokens(const float *, long, int, float *, hipStream_t))
STUB(launch_bwd_key(const BwdKeyParams &, int, int, bool, hipStream_t))
STUB(launch_dplr(const DplrParams &, int, int, int, hipStream_t))
STUB(launch_dplr_key(const DplrKeyParams &, int, int, hipStream_t))
STUB(launch_dplr_step(const DplrStepParams &, int, int, int, int, hipStream_t))
STUB(launch_dplr_decode(const DplrDecodeParams &, int, int, int, int, hipStream_t))
STUB(launch_fwd_fused(const FwdParams &, int, int, int, int, bool, hipStream_t))
STUB(launch_fwd_pipe(const FwdParams &, int, bool, hipStream_t))
STUB(launch_key_prep(const KeyPrepParams &, long, bool, hipStream_t))
STUB(launch_key_window(const FwdParams &, const KeyPrepParams &, long, int, bool, hipStream_t))
int device_cus() { return 256; }
STUB(launch_seq_order(const int32_t *, int, int32_t *, hipStream_t))
STUB(launch_recurrent_step(const StepParams &, int, int, int, int, bool, hipStream_t))
STUB(launch_decode(const DecodeParams &, int, int, int, int, bool, hipStream_t))
}  // namespace gdn

static int failures = 0;
static void expect(const char *what, long got, long want) {
  if (got != want) {
    fprintf(stderr, "%s: got %ld, want %ld\n", what, got, want);
    ++failures;
  }
}
static const void *fake(int i, int off = 0) { return (const void *)(uintptr_t)(0x1000000u * (i + 1) + off); }

static gdn_fwd_args fwd_args() {
  gdn_fwd_args a;
  memset(&a, 0, sizeof a);
  a.B = 2, a.T = 128, a.H = 4, a.d_k = 128, a.d_v = 128, a.chunk = 64, a.N = 2;
  a.dtype = GDN_BF16, a.gate = GDN_GATE_HEAD, a.write = GDN_WRITE_DELTA;
  a.q = fake(0), a.k = fake(1), a.v = fake(2), a.beta = (const float *)fake(3), a.log_alpha = (const float *)fake(4);
  a.o = (void *)fake(5), a.final_state = (float *)fake(6);
  return a;
}

int main() {
  expect("version nonzero", gdn_version() > 0, 1);
  for (int s = -6; s <= 1; ++s) expect("status string", gdn_status_str(s) != nullptr, 1);
  // forward: rejected arguments
  expect("fwd NULL", gdn_fwd_chunked(nullptr, nullptr), GDN_ERR_INVALID_ARG);
  gdn_fwd_args a = fwd_args();
  a.chunk = 32;
  expect("fwd chunk 32", gdn_fwd_chunked(&a, nullptr), GDN_ERR_UNSUPPORTED);
  a = fwd_args(), a.d_k = 96;
  expect("fwd d_k 96", gdn_fwd_chunked(&a, nullptr), GDN_ERR_UNSUPPORTED);
  a = fwd_args(), a.q = nullptr;
  expect("fwd q NULL", gdn_fwd_chunked(&a, nullptr), GDN_ERR_INVALID_ARG);
  a = fwd_args(), a.k = fake(1, 8);
  expect("fwd k misaligned", gdn_fwd_chunked(&a, nullptr), GDN_ERR_INVALID_ARG);
  a = fwd_args(), a.N = 3;
  expect("fwd N != B", gdn_fwd_chunked(&a, nullptr), GDN_ERR_INVALID_ARG);
  a = fwd_args(), a.gate = GDN_GATE_KEY;
  expect("fwd key gate without workspace", gdn_fwd_chunked(&a, nullptr), GDN_ERR_WORKSPACE);
  expect("fwd key workspace size", gdn_fwd_workspace_size(&a) > 0, 1);
  a = fwd_args(), a.B = 1, a.T = 256, a.N = 5, a.cu_seqlens = (const int32_t *)fake(7);
  expect("fwd varlen workspace size", gdn_fwd_workspace_size(&a) > 0, 1);
  expect("fwd varlen without workspace", gdn_fwd_chunked(&a, nullptr), GDN_ERR_WORKSPACE);
  a = fwd_args(), a.H = 0;
  expect("fwd workspace size of rejected args", (long)gdn_fwd_workspace_size(&a), 0);
  expect("fwd static NULL", gdn_fwd_chunked_static(nullptr, nullptr), GDN_ERR_INVALID_ARG);
  a = fwd_args(), a.d_v = 96;
  expect("fwd static d_v 96", gdn_fwd_chunked_static(&a, nullptr), GDN_ERR_UNSUPPORTED);
  // decode entry points
  expect("step NULL", gdn_fwd_recurrent_step(nullptr, nullptr), GDN_ERR_INVALID_ARG);
  gdn_step_args s;
  memset(&s, 0, sizeof s);
  s.N = 4, s.H = 2, s.d_k = 128, s.d_v = 128, s.dtype = GDN_BF16, s.gate = GDN_GATE_HEAD;
  s.q = fake(0), s.k = fake(1), s.v = fake(2), s.beta = (const float *)fake(3);
  s.state = (float *)fake(5), s.o = (void *)fake(6);
  expect("step without decays", gdn_fwd_recurrent_step(&s, nullptr), GDN_ERR_INVALID_ARG);
  expect("decode NULL", gdn_fwd_decode(nullptr, nullptr), GDN_ERR_INVALID_ARG);
  expect("dplr step NULL", gdn_fwd_dplr_step(nullptr, nullptr), GDN_ERR_INVALID_ARG);
  expect("dplr decode NULL", gdn_fwd_dplr_decode(nullptr, nullptr), GDN_ERR_INVALID_ARG);
  // gradients
  expect("bwd NULL", gdn_bwd_chunked(nullptr, nullptr), GDN_ERR_INVALID_ARG);
  gdn_bwd_args g;
  memset(&g, 0, sizeof g);
  g.B = 2, g.T = 128, g.H = 4, g.d_k = 128, g.d_v = 128, g.chunk = 64, g.N = 2;
  g.dtype = GDN_BF16, g.gate = GDN_GATE_HEAD, g.write = GDN_WRITE_DELTA;
  g.q = fake(0), g.k = fake(1), g.v = fake(2), g.beta = (const float *)fake(3), g.log_alpha = (const float *)fake(4);
  g.dout = fake(5), g.dq = (void *)fake(6), g.dk = (void *)fake(7), g.dv = (void *)fake(8);
  g.dbeta = (float *)fake(9), g.dlog_alpha = (float *)fake(10);
  expect("bwd workspace size", gdn_bwd_workspace_size(&g) > 0, 1);
  expect("bwd without workspace", gdn_bwd_chunked(&g, nullptr), GDN_ERR_WORKSPACE);
  g.gate = GDN_GATE_KEY;
  expect("bwd key workspace size", gdn_bwd_workspace_size(&g) > 0, 1);
  expect("bwd key without workspace", gdn_bwd_chunked(&g, nullptr), GDN_ERR_WORKSPACE);
  g.dq = nullptr;
  expect("bwd workspace size of rejected args", (long)gdn_bwd_workspace_size(&g), 0);
  // diagonal plus low rank
  expect("dplr NULL", gdn_fwd_dplr(nullptr, nullptr), GDN_ERR_INVALID_ARG);
  gdn_dplr_args d;
  memset(&d, 0, sizeof d);
  d.B = 2, d.T = 128, d.H = 4, d.d_k = 128, d.d_v = 128, d.chunk = 64, d.N = 2, d.dtype = GDN_BF16;
  d.gate = GDN_GATE_KEY;
  d.q = fake(0), d.k = fake(1), d.a = fake(2), d.b = fake(3), d.v = fake(4), d.log_alpha = (const float *)fake(5);
  d.o = (void *)fake(6);
  expect("dplr key workspace size", gdn_dplr_workspace_size(&d) > 0, 1);
  expect("dplr key without workspace", gdn_fwd_dplr(&d, nullptr), GDN_ERR_WORKSPACE);
  d.dtype = GDN_F32;
  expect("dplr fp32 d_k 128", gdn_fwd_dplr(&d, nullptr), GDN_ERR_UNSUPPORTED);
  // out-of-range enum values, as a C caller may store them, are rejected
  gdn_fwd_args e = fwd_args();
  int seven = 7;
  memcpy(&e.gate, &seven, sizeof seven);
  expect("fwd gate 7", gdn_fwd_chunked(&e, nullptr), GDN_ERR_INVALID_ARG);
  e = fwd_args();
  memcpy(&e.dtype, &seven, sizeof seven);
  expect("fwd dtype 7", gdn_fwd_chunked(&e, nullptr), GDN_ERR_INVALID_ARG);
  gdn_bwd_args ge = g;
  memcpy(&ge.write, &seven, sizeof seven);
  expect("bwd write 7", gdn_bwd_chunked(&ge, nullptr), GDN_ERR_INVALID_ARG);
  gdn_dplr_args de = d;
  memcpy(&de.gate, &seven, sizeof seven);
  expect("dplr gate 7", gdn_fwd_dplr(&de, nullptr), GDN_ERR_INVALID_ARG);
  gdn_step_args se = s;
  memcpy(&se.dtype, &seven, sizeof seven);
  expect("step dtype 7", gdn_fwd_recurrent_step(&se, nullptr), GDN_ERR_INVALID_ARG);
  expect("launches reached", launches, 0);
  if (failures == 0) printf("boundary sanitizer run: clean\n");
  return failures ? 1 : 0;
}
