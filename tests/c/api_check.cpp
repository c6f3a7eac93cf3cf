// api_check.cpp -- drives the host-side argument validation of libgdn's C ABI (include/gdn.h)
// so that it can run under AddressSanitizer and UndefinedBehaviorSanitizer on a machine
// without a GPU.  Every call here is rejected on the host (or, for a well-formed call, fails
// at the launch because there is no device); none touches memory through the fake pointers.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../include/gdn.h"

static int fails = 0;
#define EXPECT(expr, want)                                                                     \
  do {                                                                                         \
    const int got_ = (int)(expr);                                                              \
    if (got_ != (int)(want)) {                                                                 \
      fprintf(stderr, "FAIL line %d: %s -> %d, expected %d\n", __LINE__, #expr, got_, (int)(want)); \
      ++fails;                                                                                 \
    }                                                                                          \
  } while (0)

static void* P(uintptr_t off) { return reinterpret_cast<void*>(uintptr_t(0x10000) + off); }

static gdn_chunk_desc_t desc(int64_t T = 64, int32_t chunk = 64, int64_t every = 0) {
  gdn_chunk_desc_t d;
  memset(&d, 0, sizeof d);
  d.B = 1; d.H = 2; d.T = T; d.Dk = 128; d.Dv = 128; d.chunk = chunk;
  d.in_dtype = GDN_BF16; d.out_dtype = GDN_BF16; d.ckpt_every = every;
  return d;
}

static gdn_status_t fwd(int kda, const gdn_chunk_desc_t* d, uintptr_t o_off = 0x6000000, void* s_ckpt = nullptr,
                        void* ws = nullptr, size_t ws_bytes = 0) {
  auto f = kda ? kda_chunk_fwd : gdn_chunk_fwd;
  return f(d, P(0), P(0x1000000), P(0x2000000), P(0x3000000), P(0x4000000), (const float*)P(0x5000000),
           P(o_off), (float*)P(0x7000000), (float*)s_ckpt, ws, ws_bytes, nullptr);
}

int main() {
  const gdn_status_t INV = GDN_ERROR_INVALID_VALUE, NS = GDN_ERROR_NOT_SUPPORTED;
  for (int kda = 0; kda < 2; ++kda) {
    EXPECT(fwd(kda, nullptr), INV);
    gdn_chunk_desc_t d = desc(64, 48);
    EXPECT(fwd(kda, &d), INV);
    d = desc(-1);
    EXPECT(fwd(kda, &d), INV);
    d = desc(); d.Dk = 0;
    EXPECT(fwd(kda, &d), INV);
    d = desc(); d.Dv = 64;
    EXPECT(fwd(kda, &d), NS);
    d = desc(); d.Dk = d.Dv = 96;
    EXPECT(fwd(kda, &d), NS);
    d = desc(); d.in_dtype = (gdn_dtype_t)7;
    EXPECT(fwd(kda, &d), INV);
    d = desc(); d.B = INT64_C(1) << 40; d.H = INT64_C(1) << 30;
    EXPECT(fwd(kda, &d), INV);
    d = desc(128, 64, 32);  // snapshots not a multiple of the chunk
    EXPECT(fwd(kda, &d), INV);
    d = desc(128, 64, 64);  // snapshots requested, no buffer
    EXPECT(fwd(kda, &d), INV);
    d = desc();
    EXPECT(fwd(kda, &d, 0x6000008), INV);  // o misaligned
    EXPECT(fwd(kda, &d, 0x5000000), INV);  // o overlaps s0
    d = desc(128, 64, 64);                 // snapshot buffer the runtime cannot describe
    EXPECT(fwd(kda, &d, 0x6000000, P(0x8000000)), INV);
    d = desc();
    if (kda) EXPECT(fwd(kda, &d, 0x6000000, nullptr, P(0x9000000), 16), INV);  // workspace too small
  }
  // the allocation-free KDA prefill validates like kda_chunk_fwd
  {
    gdn_chunk_desc_t d = desc(64, 48);
    EXPECT(kda_chunk_fwd_noalloc(nullptr, P(0), P(0x1000000), P(0x2000000), P(0x3000000), P(0x4000000), nullptr,
                                 P(0x6000000), nullptr, nullptr, nullptr), INV);
    EXPECT(kda_chunk_fwd_noalloc(&d, P(0), P(0x1000000), P(0x2000000), P(0x3000000), P(0x4000000), nullptr,
                                 P(0x6000000), nullptr, nullptr, nullptr), INV);
    d = desc();
    EXPECT(kda_chunk_fwd_noalloc(&d, P(0), P(0x1000000), P(0x2000000), P(0x3000000), P(0x4000000), nullptr,
                                 P(0x6000008), nullptr, nullptr, nullptr), INV);  // o misaligned
    d = desc(128, 64, 64);
    EXPECT(kda_chunk_fwd_noalloc(&d, P(0), P(0x1000000), P(0x2000000), P(0x3000000), P(0x4000000), nullptr,
                                 P(0x6000000), nullptr, nullptr, nullptr), INV);  // snapshots without a buffer
  }
  size_t n = 0;
  gdn_chunk_desc_t d = desc(200);
  EXPECT(gdn_chunk_workspace_size(&d, 0, &n), GDN_SUCCESS);
  EXPECT(n == 0, 1);
  EXPECT(gdn_chunk_workspace_size(&d, 1, &n), GDN_SUCCESS);
  EXPECT(n > 0, 1);
  EXPECT(gdn_chunk_workspace_size(nullptr, 0, &n), INV);
  EXPECT(gdn_chunk_workspace_size(&d, 0, nullptr), INV);

  // decode step
  EXPECT(gdn_decode_step(-1, 2, 128, 128, GDN_BF16, GDN_BF16, (float*)P(0), P(0x100000), P(0x200000), P(0x300000),
                         P(0x400000), P(0x500000), P(0x600000), nullptr), INV);
  EXPECT(gdn_decode_step(4, 2, 128, 64, GDN_BF16, GDN_BF16, (float*)P(0), P(0x100000), P(0x200000), P(0x300000),
                         P(0x400000), P(0x500000), P(0x600000), nullptr), NS);
  EXPECT(gdn_decode_step(4, 2, 96, 96, GDN_BF16, GDN_BF16, (float*)P(0), P(0x100000), P(0x200000), P(0x300000),
                         P(0x400000), P(0x500000), P(0x600000), nullptr), NS);
  EXPECT(gdn_decode_step(4, 2, 128, 128, GDN_BF16, GDN_BF16, (float*)P(4), P(0x100000), P(0x200000), P(0x300000),
                         P(0x400000), P(0x500000), P(0x600000), nullptr), INV);
  EXPECT(gdn_decode_step(4, 2, 128, 128, GDN_BF16, GDN_BF16, (float*)P(0), nullptr, P(0x200000), P(0x300000),
                         P(0x400000), P(0x500000), P(0x600000), nullptr), INV);
  EXPECT(gdn_decode_step(4, 2, 128, 128, GDN_BF16, GDN_BF16, (float*)P(0), P(0x100000), P(0x200000), P(0x300000),
                         P(0x400000), P(0x500000), P(0x100), nullptr), INV);  // o inside the state
  EXPECT(gdn_decode_step(0, 2, 128, 128, GDN_BF16, GDN_BF16, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                         nullptr, nullptr), GDN_SUCCESS);

  // serving decode window
  gdn_decode_ex_desc_t e;
  memset(&e, 0, sizeof e);
  e.N = 4; e.H = 4; e.H_qk = 2; e.Dk = e.Dv = 128; e.T = 2; e.P = 8;
  e.in_dtype = GDN_BF16; e.out_dtype = GDN_BF16; e.write_state = 1;
  auto dex = [&](const gdn_decode_ex_desc_t* dd, void* o) {
    return gdn_decode_ex(dd, (float*)P(0), nullptr, P(0x1000000), P(0x2000000), P(0x3000000), P(0x4000000),
                         P(0x5000000), nullptr, nullptr, nullptr, o, nullptr);
  };
  EXPECT(dex(nullptr, P(0x6000000)), INV);
  gdn_decode_ex_desc_t e2 = e; e2.H_qk = 3;
  EXPECT(dex(&e2, P(0x6000000)), INV);
  e2 = e; e2.kda = 1; e2.raw_gates = 1;
  EXPECT(dex(&e2, P(0x6000000)), NS);
  e2 = e; e2.write_state = 2;
  EXPECT(dex(&e2, P(0x6000000)), INV);
  e2 = e; e2.P = 2;
  EXPECT(dex(&e2, P(0x6000000)), INV);  // no slot table and fewer pool rows than sequences
  e2 = e; e2.raw_gates = 1;
  EXPECT(dex(&e2, P(0x6000000)), INV);  // raw gates without A_log / dt_bias
  EXPECT(dex(&e, P(0x100)), INV);       // o inside the pool
  e2 = e; e2.write_state = 0;
  EXPECT(dex(&e2, nullptr), GDN_SUCCESS);  // verify without outputs: nothing to do

  // prefill with the layer prologue
  gdn_chunk_ex_desc_t x;
  memset(&x, 0, sizeof x);
  x.base = desc();
  x.H_qk = 3;
  auto fex = [&](const gdn_chunk_ex_desc_t* dd, const float* A_log, const int32_t* cu) {
    return gdn_chunk_fwd_ex(dd, P(0), P(0x1000000), P(0x2000000), P(0x3000000), P(0x4000000), A_log,
                            (const float*)P(0xa000000), cu, nullptr, P(0x6000000), (float*)P(0x7000000), nullptr,
                            nullptr);
  };
  EXPECT(fex(&x, nullptr, nullptr), INV);  // H not a multiple of H_qk
  x.H_qk = 1; x.raw_gates = 1;
  EXPECT(fex(&x, nullptr, nullptr), INV);  // raw gates need A_log
  x.raw_gates = 0; x.qk_l2norm = 3;
  EXPECT(fex(&x, nullptr, nullptr), INV);
  x.qk_l2norm = 0; x.base.ckpt_every = 64;
  EXPECT(fex(&x, nullptr, (const int32_t*)P(0xb000000)), NS);  // ragged batches take no snapshots
  x.base = desc(); x.base.Dk = x.base.Dv = 64; x.H_qk = 1; x.qk_l2norm = 1;
  EXPECT(fex(&x, nullptr, nullptr), NS);  // the prologue runs on the matrix-core path only

  for (int s = 0; s < 5; ++s) EXPECT(gdn_status_string((gdn_status_t)s) != nullptr, 1);
  EXPECT(gdn_version(), GDN_VERSION);
  if (fails) {
    fprintf(stderr, "%d check(s) failed\n", fails);
    return 1;
  }
  printf("api_check: all checks passed\n");
  return 0;
}
