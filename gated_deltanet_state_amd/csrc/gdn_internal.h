// gdn_internal.h -- launch descriptors shared by the host API and the HIP kernels of
// libgdn.so.  Not part of the public ABI (include/gdn.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gdn.h"

namespace gdn {

// One chunkwise prefill call after host-side validation.
struct ChunkArgs {
  int64_t B, H, T, D;      // Dk == Dv == D
  int chunk;
  gdn_dtype_t in_dtype, out_dtype;
  int64_t ckpt_every;      // 0 = none
  int64_t n_ckpt;          // snapshots per stream = T / ckpt_every (0 when disabled)
  const void *q, *k, *v, *beta, *log_alpha;
  const float* s0;         // may be null
  void* o;
  float* s_final;          // may be null
  float* s_ckpt;           // may be null iff n_ckpt == 0
  // layer prologue (gdn_chunk_fwd_ex; matrix-core path only)
  int64_t Hqk;             // query/key heads (H a multiple); equals H for the plain entry points
  int raw_gates;           // beta / log_alpha carry the raw b / a projections
  int qk_l2norm;           // q and k rows are scaled to unit length in the kernel
  const float *A_log, *dt_bias;  // [H], raw gates only
  const int32_t* cu_seqlens;     // [B + 1] token offsets of a ragged batch (T = total), or null
  void* workspace;               // caller's device workspace (KDA two-kernel form), or null
  size_t workspace_bytes;
};

struct DecodeArgs {
  int64_t N, H, D;
  gdn_dtype_t in_dtype, out_dtype;
  float* state;
  const void *q, *k, *v, *beta, *log_alpha;
  void* o;
};

// Serving-side decode window (see gdn_decode_ex in gdn.h), after host-side validation.
struct DecodeExArgs {
  int64_t N, H, Hqk, D, T, P;  // P: rows of the state pool
  gdn_dtype_t in_dtype, out_dtype;
  int kda, qk_l2norm, raw_gates, write_state;
  float* pool;
  const int32_t* slots;     // may be null (slot n = n)
  const int32_t* n_commit;  // may be null (all T tokens)
  const void *q, *k, *v, *beta, *log_alpha;
  const float *A_log, *dt_bias;  // raw gates only
  void* o;                  // may be null
};

// Matrix-core prefill (bf16 inputs, D = 128, chunk = 64).
bool chunk_mfma_supported(const ChunkArgs& a);
hipError_t launch_chunk_mfma(const ChunkArgs& a, bool kda, hipStream_t stream);
hipError_t launch_kda_mfma(const ChunkArgs& a, hipStream_t stream);
// Workspace of the two-kernel matrix-core KDA prefill: one 64 KiB record per (stream, chunk)
// for the whole call.  A smaller workspace of at least two records is used slab by slab.
size_t kda_workspace_bytes(const ChunkArgs& a);
bool kda_slabs_fit(const ChunkArgs& a, size_t bytes);
constexpr size_t kKdaMinWorkspace = (size_t)2 << 16;
// Device address and size of the fixed scratch used by the allocation-free KDA entry point.
hipError_t kda_scratch(void** ptr, size_t* bytes);

// fp32 vector-unit prefill (fp32 or bf16 inputs, D in {16,32,64,128}, chunk in {16,32,64}).
bool chunk_valu_supported(const ChunkArgs& a);
hipError_t launch_chunk_valu(const ChunkArgs& a, bool kda, hipStream_t stream);

// Decode step (D in {16,32,64,128}).
bool decode_supported(const DecodeArgs& a);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_ex(const DecodeExArgs& a, hipStream_t stream);

}  // namespace gdn
