// gdn_api.cpp -- the extern "C" entry points of libgdn.so: synchronous host-side
// validation, then dispatch to the kernel launches on the caller's stream (one, except the
// matrix-core KDA prefill with a workspace: two per slab of the workspace).
//
// Nothing here touches device memory or synchronises.  The HIP calls made during validation
// are the pointer-attribute query on a snapshot buffer (is it device memory or pinned host
// memory?) and, for kda_chunk_fwd_noalloc, the device address of its static scratch (taken
// once per device).  Every check, those included, runs before any launch, so a rejected call
// has launched nothing.
#include <stdint.h>
#include <string.h>

#include "gdn_internal.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool aligned_elem(const void* p, gdn_dtype_t dt) {
  const uintptr_t m = dt == GDN_F32 ? 3u : 1u;
  return (reinterpret_cast<uintptr_t>(p) & m) == 0;
}

// A dtype field or argument is checked through its integer bits: a caller can pass any int,
// and reading an out-of-range value as the enum type is undefined behaviour in C++.
bool valid_dtype(const gdn_dtype_t& d) {
  int v;
  memcpy(&v, &d, sizeof v);
  return v == GDN_F32 || v == GDN_BF16;
}
static_assert(sizeof(gdn_dtype_t) == sizeof(int), "gdn_dtype_t is an int");

// Byte ranges [a, a + na) and [b, b + nb) intersect.
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return na > 0 && nb > 0 && x < y + nb && y < x + na;
}

// Product of non-negative sizes with an overflow guard against 2^62.
bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > (INT64_C(1) << 62) / a) return false;
  *out = a * b;
  return true;
}

gdn_status_t check_chunk_desc(const gdn_chunk_desc_t* d, int is_kda, gdn::ChunkArgs* out) {
  if (!d) return GDN_ERROR_INVALID_VALUE;
  if (d->B < 0 || d->H < 0 || d->T < 0 || d->Dk <= 0 || d->Dv <= 0) return GDN_ERROR_INVALID_VALUE;
  if (!valid_dtype(d->in_dtype) || !valid_dtype(d->out_dtype)) return GDN_ERROR_INVALID_VALUE;
  if (d->chunk != 16 && d->chunk != 32 && d->chunk != 64) return GDN_ERROR_INVALID_VALUE;
  if (d->ckpt_every < 0 || (d->ckpt_every > 0 && d->ckpt_every % d->chunk != 0))
    return GDN_ERROR_INVALID_VALUE;
  int64_t tmp;
  if (!mul_ok(d->B, d->H, &tmp) || !mul_ok(tmp, d->T, &tmp) || !mul_ok(tmp, d->Dk + d->Dv, &tmp))
    return GDN_ERROR_INVALID_VALUE;
  if (d->Dk != d->Dv) return GDN_ERROR_NOT_SUPPORTED;
  gdn::ChunkArgs a;
  memset(&a, 0, sizeof a);
  a.B = d->B; a.H = d->H; a.T = d->T; a.D = d->Dk; a.chunk = d->chunk;
  a.in_dtype = d->in_dtype; a.out_dtype = d->out_dtype; a.ckpt_every = d->ckpt_every;
  a.n_ckpt = d->ckpt_every > 0 ? d->T / d->ckpt_every : 0;
  a.Hqk = d->H;  // one query/key head per value head unless gdn_chunk_fwd_ex says otherwise
  (void)is_kda;
  if (!gdn::chunk_mfma_supported(a) && !gdn::chunk_valu_supported(a)) return GDN_ERROR_NOT_SUPPORTED;
  *out = a;
  return GDN_SUCCESS;
}

// Layer prologue of gdn_chunk_fwd_ex (NULL for the plain entry points).
struct Prologue {
  int64_t H_qk;
  int raw_gates;
  int qk_l2norm;
  const float *A_log, *dt_bias;
  const int32_t* cu_seqlens;  // ragged batch: [B + 1] token offsets, T = total tokens
};

gdn_status_t chunk_fwd(int is_kda, const gdn_chunk_desc_t* d, const void* q, const void* k,
                       const void* v, const void* beta, const void* log_alpha, const float* s0,
                       void* o, float* s_final, float* s_ckpt, void* workspace,
                       size_t workspace_bytes, void* stream, const Prologue* pro = nullptr,
                       bool use_scratch = false) {
  gdn::ChunkArgs a;
  gdn_status_t st = check_chunk_desc(d, is_kda, &a);
  if (st != GDN_SUCCESS) return st;
  if (pro) {
    if (pro->H_qk <= 0 || a.H % pro->H_qk != 0) return GDN_ERROR_INVALID_VALUE;
    if (pro->raw_gates != 0 && pro->raw_gates != 1) return GDN_ERROR_INVALID_VALUE;
    if (pro->qk_l2norm != 0 && pro->qk_l2norm != 1) return GDN_ERROR_INVALID_VALUE;
    // the prologue runs in the matrix-core kernel only; without one, the plain paths apply
    if ((pro->H_qk != a.H || pro->raw_gates || pro->qk_l2norm || pro->cu_seqlens) &&
        !gdn::chunk_mfma_supported(a))
      return GDN_ERROR_NOT_SUPPORTED;
    if (pro->cu_seqlens) {
      if (a.ckpt_every != 0) return GDN_ERROR_NOT_SUPPORTED;  // snapshots need a common length
      if (!aligned_elem(pro->cu_seqlens, GDN_F32)) return GDN_ERROR_INVALID_VALUE;
      a.cu_seqlens = pro->cu_seqlens;
    }
    if (pro->raw_gates && (!pro->A_log || !pro->dt_bias || !aligned_elem(pro->A_log, GDN_F32) ||
                           !aligned_elem(pro->dt_bias, GDN_F32)))
      return GDN_ERROR_INVALID_VALUE;
    a.Hqk = pro->H_qk;
    a.raw_gates = pro->raw_gates;
    a.qk_l2norm = pro->qk_l2norm;
    a.A_log = pro->raw_gates ? pro->A_log : nullptr;
    a.dt_bias = pro->raw_gates ? pro->dt_bias : nullptr;
  }
  // Only the matrix-core KDA prefill takes a workspace (its two-kernel form); without one it
  // runs as a single kernel.  A workspace that holds every record of the call is used in one
  // slab; a smaller one (at least two records) slab by slab.
  if (workspace && is_kda && gdn::chunk_mfma_supported(a) && a.T > 0) {
    if (!aligned16(workspace) || workspace_bytes < gdn::kKdaMinWorkspace) return GDN_ERROR_INVALID_VALUE;
    a.workspace = workspace;
    a.workspace_bytes = workspace_bytes;
  }
  const int64_t BH = a.B * a.H;
  if (BH == 0) return GDN_SUCCESS;
  const size_t state_bytes = (size_t)BH * (size_t)(a.D * a.D) * sizeof(float);
  const size_t in_elem = a.in_dtype == GDN_F32 ? 4 : 2;
  const size_t out_elem = a.out_dtype == GDN_F32 ? 4 : 2;
  // a ragged batch packs all sequences into H * T rows (T = total tokens)
  const size_t o_rows = a.cu_seqlens ? (size_t)a.H * (size_t)a.T : (size_t)BH * (size_t)a.T;
  const size_t o_bytes = o_rows * (size_t)a.D * out_elem;
  if (a.T > 0) {
    if (!q || !k || !v || !beta || !log_alpha || !o) return GDN_ERROR_INVALID_VALUE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return GDN_ERROR_INVALID_VALUE;
    if (!aligned_elem(beta, a.in_dtype) || !aligned_elem(log_alpha, a.in_dtype))
      return GDN_ERROR_INVALID_VALUE;
    if (is_kda && !aligned16(log_alpha)) return GDN_ERROR_INVALID_VALUE;
  }
  if (s0 && !aligned16(s0)) return GDN_ERROR_INVALID_VALUE;
  if (s_final && !aligned16(s_final)) return GDN_ERROR_INVALID_VALUE;
  if (a.n_ckpt > 0) {
    if (!s_ckpt || !aligned16(s_ckpt)) return GDN_ERROR_INVALID_VALUE;
    // Snapshots may go to pinned host memory: the kernel then writes each one into host RAM
    // as it is reached, with no copy and no synchronisation.  Pageable host memory, which the
    // GPU cannot write, is rejected, and so is a pointer the runtime cannot describe: storing
    // through it could fault the GPU.
    hipPointerAttribute_t at;
    if (hipPointerGetAttributes(&at, s_ckpt) != hipSuccess) {
      (void)hipGetLastError();  // the failed query must not be reported by a later call
      return GDN_ERROR_INVALID_VALUE;
    }
    if (at.type != hipMemoryTypeDevice && at.type != hipMemoryTypeManaged && at.type != hipMemoryTypeHost)
      return GDN_ERROR_INVALID_VALUE;
    if (at.type == hipMemoryTypeHost) {
      if (!at.devicePointer || !aligned16(at.devicePointer)) return GDN_ERROR_INVALID_VALUE;
      s_ckpt = static_cast<float*>(at.devicePointer);
    }
  } else {
    s_ckpt = nullptr;
  }
  // s_final may be s0 exactly (in place); any other overlap among the state buffers or
  // with o is rejected.
  if (s0 && s_final && (const void*)s0 != (const void*)s_final &&
      overlaps(s0, state_bytes, s_final, state_bytes))
    return GDN_ERROR_INVALID_VALUE;
  const size_t ck_bytes = (size_t)a.n_ckpt * state_bytes;
  if (s_ckpt && (overlaps(s_ckpt, ck_bytes, s0, s0 ? state_bytes : 0) ||
                 overlaps(s_ckpt, ck_bytes, s_final, s_final ? state_bytes : 0) ||
                 overlaps(s_ckpt, ck_bytes, o, o_bytes)))
    return GDN_ERROR_INVALID_VALUE;
  if (o && (overlaps(o, o_bytes, s0, s0 ? state_bytes : 0) ||
            overlaps(o, o_bytes, s_final, s_final ? state_bytes : 0)))
    return GDN_ERROR_INVALID_VALUE;
  if (a.workspace && (overlaps(a.workspace, a.workspace_bytes, o, o_bytes) ||
                      overlaps(a.workspace, a.workspace_bytes, s_final, s_final ? state_bytes : 0) ||
                      overlaps(a.workspace, a.workspace_bytes, s0, s0 ? state_bytes : 0) ||
                      overlaps(a.workspace, a.workspace_bytes, s_ckpt, s_ckpt ? ck_bytes : 0)))
    return GDN_ERROR_INVALID_VALUE;
  if (a.workspace) {  // the preparation kernel writes the workspace while it reads the inputs
    const size_t tok = (size_t)BH * (size_t)a.T;
    const size_t qkv_bytes = tok * (size_t)a.D * in_elem;
    const size_t la_bytes = tok * (is_kda ? (size_t)a.D : 1) * in_elem;
    if (overlaps(a.workspace, a.workspace_bytes, q, qkv_bytes) || overlaps(a.workspace, a.workspace_bytes, k, qkv_bytes) ||
        overlaps(a.workspace, a.workspace_bytes, v, qkv_bytes) ||
        overlaps(a.workspace, a.workspace_bytes, beta, tok * in_elem) ||
        overlaps(a.workspace, a.workspace_bytes, log_alpha, la_bytes))
      return GDN_ERROR_INVALID_VALUE;
  }

  a.q = q; a.k = k; a.v = v; a.beta = beta; a.log_alpha = log_alpha;
  a.s0 = s0; a.o = o; a.s_final = s_final; a.s_ckpt = s_ckpt;
  if (use_scratch && is_kda && gdn::chunk_mfma_supported(a) && a.T > 0) {
    // the allocation-free entry point: the library's fixed device scratch as the workspace
    if (gdn::kda_scratch(&a.workspace, &a.workspace_bytes) != hipSuccess) {
      (void)hipGetLastError();
      return GDN_ERROR_HIP;
    }
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = gdn::chunk_mfma_supported(a) ? gdn::launch_chunk_mfma(a, is_kda != 0, s)
                          : gdn::launch_chunk_valu(a, is_kda != 0, s);
  return e == hipSuccess ? GDN_SUCCESS : GDN_ERROR_HIP;
}

}  // namespace

extern "C" {

gdn_status_t gdn_chunk_workspace_size(const gdn_chunk_desc_t* d, int is_kda, size_t* bytes) {
  if (!bytes) return GDN_ERROR_INVALID_VALUE;
  gdn::ChunkArgs a;
  gdn_status_t st = check_chunk_desc(d, is_kda, &a);
  if (st != GDN_SUCCESS) return st;
  *bytes = (is_kda && gdn::chunk_mfma_supported(a)) ? gdn::kda_workspace_bytes(a) : 0;
  return GDN_SUCCESS;
}

gdn_status_t gdn_chunk_fwd(const gdn_chunk_desc_t* d, const void* q, const void* k, const void* v,
                           const void* beta, const void* log_alpha, const float* s0, void* o,
                           float* s_final, float* s_ckpt, void* workspace, size_t workspace_bytes,
                           void* stream) {
  return chunk_fwd(0, d, q, k, v, beta, log_alpha, s0, o, s_final, s_ckpt, workspace,
                   workspace_bytes, stream);
}

gdn_status_t kda_chunk_fwd(const gdn_chunk_desc_t* d, const void* q, const void* k, const void* v,
                           const void* beta, const void* log_alpha, const float* s0, void* o,
                           float* s_final, float* s_ckpt, void* workspace, size_t workspace_bytes,
                           void* stream) {
  return chunk_fwd(1, d, q, k, v, beta, log_alpha, s0, o, s_final, s_ckpt, workspace,
                   workspace_bytes, stream);
}

gdn_status_t kda_chunk_fwd_noalloc(const gdn_chunk_desc_t* d, const void* q, const void* k, const void* v,
                                   const void* beta, const void* log_alpha, const float* s0, void* o,
                                   float* s_final, float* s_ckpt, void* stream) {
  return chunk_fwd(1, d, q, k, v, beta, log_alpha, s0, o, s_final, s_ckpt, nullptr, 0, stream, nullptr, true);
}

gdn_status_t gdn_chunk_fwd_ex(const gdn_chunk_ex_desc_t* d, const void* q, const void* k, const void* v,
                              const void* beta, const void* log_alpha, const float* A_log,
                              const float* dt_bias, const int32_t* cu_seqlens, const float* s0, void* o,
                              float* s_final, float* s_ckpt, void* stream) {
  if (!d) return GDN_ERROR_INVALID_VALUE;
  const Prologue pro = {d->H_qk, d->raw_gates, d->qk_l2norm, A_log, dt_bias, cu_seqlens};
  return chunk_fwd(0, &d->base, q, k, v, beta, log_alpha, s0, o, s_final, s_ckpt, nullptr, 0, stream, &pro);
}

gdn_status_t gdn_decode_step(int64_t N, int64_t H, int64_t Dk, int64_t Dv, gdn_dtype_t in_dtype,
                             gdn_dtype_t out_dtype, float* state, const void* q, const void* k,
                             const void* v, const void* beta, const void* log_alpha, void* o,
                             void* stream) {
  if (N < 0 || H < 0 || Dk <= 0 || Dv <= 0) return GDN_ERROR_INVALID_VALUE;
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return GDN_ERROR_INVALID_VALUE;
  int64_t tmp;
  if (!mul_ok(N, H, &tmp) || !mul_ok(tmp, Dk * Dv, &tmp)) return GDN_ERROR_INVALID_VALUE;
  if (Dk != Dv) return GDN_ERROR_NOT_SUPPORTED;
  gdn::DecodeArgs a;
  a.N = N; a.H = H; a.D = Dk; a.in_dtype = in_dtype; a.out_dtype = out_dtype;
  if (!gdn::decode_supported(a)) return GDN_ERROR_NOT_SUPPORTED;
  if (N * H == 0) return GDN_SUCCESS;
  if (!state || !q || !k || !v || !beta || !log_alpha || !o) return GDN_ERROR_INVALID_VALUE;
  if (!aligned16(state) || !aligned_elem(q, in_dtype) || !aligned_elem(k, in_dtype) ||
      !aligned_elem(v, in_dtype) || !aligned_elem(beta, in_dtype) ||
      !aligned_elem(log_alpha, in_dtype) || !aligned_elem(o, out_dtype))
    return GDN_ERROR_INVALID_VALUE;
  const size_t state_bytes = (size_t)(N * H) * (size_t)(Dk * Dv) * sizeof(float);
  const size_t o_bytes = (size_t)(N * H) * (size_t)Dv * (out_dtype == GDN_F32 ? 4 : 2);
  if (overlaps(state, state_bytes, o, o_bytes)) return GDN_ERROR_INVALID_VALUE;
  a.state = state; a.q = q; a.k = k; a.v = v; a.beta = beta; a.log_alpha = log_alpha; a.o = o;
  hipError_t e = gdn::launch_decode(a, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? GDN_SUCCESS : GDN_ERROR_HIP;
}

gdn_status_t gdn_decode_ex(const gdn_decode_ex_desc_t* d, float* pool, const int32_t* slots,
                           const void* q, const void* k, const void* v, const void* beta,
                           const void* log_alpha, const float* A_log, const float* dt_bias,
                           const int32_t* n_commit, void* o, void* stream) {
  if (!d) return GDN_ERROR_INVALID_VALUE;
  if (d->N < 0 || d->H <= 0 || d->H_qk <= 0 || d->Dk <= 0 || d->Dv <= 0 || d->T <= 0 || d->P < 0)
    return GDN_ERROR_INVALID_VALUE;
  if (d->H % d->H_qk != 0) return GDN_ERROR_INVALID_VALUE;
  if (!valid_dtype(d->in_dtype) || !valid_dtype(d->out_dtype)) return GDN_ERROR_INVALID_VALUE;
  for (int32_t f : {d->kda, d->qk_l2norm, d->raw_gates, d->write_state})
    if (f != 0 && f != 1) return GDN_ERROR_INVALID_VALUE;
  int64_t tok, rows, tmp;
  if (!mul_ok(d->N, d->T, &tok) || !mul_ok(tok, d->H, &rows) || !mul_ok(rows, d->Dk, &tmp) ||
      !mul_ok(d->P, d->H, &tmp) || !mul_ok(tmp, d->Dk * d->Dv, &tmp))
    return GDN_ERROR_INVALID_VALUE;
  if (d->Dk != d->Dv) return GDN_ERROR_NOT_SUPPORTED;
  if (d->Dk != 16 && d->Dk != 32 && d->Dk != 64 && d->Dk != 128) return GDN_ERROR_NOT_SUPPORTED;
  if (d->kda && d->raw_gates) return GDN_ERROR_NOT_SUPPORTED;
  if (!slots && d->P < d->N) return GDN_ERROR_INVALID_VALUE;
  if (d->N == 0 || d->P == 0 || (!d->write_state && !o)) return GDN_SUCCESS;
  if (!pool || !q || !k || !v || !beta || !log_alpha) return GDN_ERROR_INVALID_VALUE;
  if (d->raw_gates && (!A_log || !dt_bias)) return GDN_ERROR_INVALID_VALUE;
  const gdn_dtype_t it = d->in_dtype;
  if (!aligned16(pool) || !aligned_elem(q, it) || !aligned_elem(k, it) || !aligned_elem(v, it) ||
      !aligned_elem(beta, it) || !aligned_elem(log_alpha, it) || (o && !aligned_elem(o, d->out_dtype)) ||
      (slots && !aligned_elem(slots, GDN_F32)) || (n_commit && !aligned_elem(n_commit, GDN_F32)) ||
      (d->raw_gates && (!aligned_elem(A_log, GDN_F32) || !aligned_elem(dt_bias, GDN_F32))))
    return GDN_ERROR_INVALID_VALUE;
  const size_t pool_bytes = (size_t)(d->P * d->H) * (size_t)(d->Dk * d->Dv) * sizeof(float);
  const size_t o_bytes = (size_t)rows * (size_t)d->Dv * (d->out_dtype == GDN_F32 ? 4 : 2);
  if (o && overlaps(pool, pool_bytes, o, o_bytes)) return GDN_ERROR_INVALID_VALUE;
  gdn::DecodeExArgs a;
  memset(&a, 0, sizeof a);
  a.N = d->N; a.H = d->H; a.Hqk = d->H_qk; a.D = d->Dk; a.T = d->T; a.P = d->P;
  a.in_dtype = d->in_dtype; a.out_dtype = d->out_dtype;
  a.kda = d->kda; a.qk_l2norm = d->qk_l2norm; a.raw_gates = d->raw_gates; a.write_state = d->write_state;
  a.pool = pool; a.slots = slots; a.n_commit = n_commit;
  a.q = q; a.k = k; a.v = v; a.beta = beta; a.log_alpha = log_alpha;
  a.A_log = d->raw_gates ? A_log : nullptr;
  a.dt_bias = d->raw_gates ? dt_bias : nullptr;
  a.o = o;
  hipError_t e = gdn::launch_decode_ex(a, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? GDN_SUCCESS : GDN_ERROR_HIP;
}

const char* gdn_status_string(gdn_status_t s) {
  switch (s) {
    case GDN_SUCCESS: return "success";
    case GDN_ERROR_INVALID_VALUE: return "invalid value (null/misaligned pointer, bad size or option, overlapping buffers)";
    case GDN_ERROR_NOT_SUPPORTED: return "combination of head size, chunk and dtypes not supported";
    case GDN_ERROR_HIP: return "HIP runtime error or kernel launch failure";
    default: return "unknown status";
  }
}

int gdn_version(void) { return GDN_VERSION; }

}  // extern "C"
