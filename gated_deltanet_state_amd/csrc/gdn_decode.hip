// gdn_decode.hip -- one recurrent step of the gated delta rule for a batch of fp32
// states, updated in place (gfx950).
//
// Per state S (D x D, row i = value channel i) and token (q, k, v, beta, alpha):
//   r_i = s_i . k        p_i = s_i . q          (one read of row i)
//   u_i = beta (v_i - alpha r_i)                (delta correction with the decayed state)
//   o_i = alpha p_i + u_i (k . q)               (the query reads the updated state)
//   s_i <- alpha s_i + u_i k^T                  (one write of row i)
// This is the gated delta rule S_t = alpha_t S_{t-1}(I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
// o_t = S_t q_t ("From Traditional Attention to hybrid ones", section 5, decay first and
// then the delta update on the decayed state) taken one token at a time.
//
// The step is bound by HBM: every state is read once and written once (8 D^2 bytes),
// against 7 D^2 flops.  Layout of the work: a group of 2D lanes owns one state; lane
// (row group rg, column quad c4) holds rows rg, rg+8, ... of columns 4c4..4c4+3 as float4,
// so each wavefront load/store instruction moves whole contiguous rows (coalesced 16-byte
// accesses).  The two row dot products are reduced across the D/4 lanes of a row with
// cross-lane shuffles; all loads of the state are issued before any reduction so that the
// whole 64 KiB state of a workgroup is in flight at once.
#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>

#include "gdn_internal.h"

namespace gdn {
namespace {

__device__ __forceinline__ float ld_in(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ld_in(const __hip_bfloat16* p, int64_t i) {
  const uint16_t b = reinterpret_cast<const uint16_t*>(p)[i];
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

__device__ __forceinline__ void st_out(float* p, int64_t i, float x) { p[i] = x; }
__device__ __forceinline__ void st_out(__hip_bfloat16* p, int64_t i, float x) {
  p[i] = __float2bfloat16(x);  // round to nearest even
}

// Sum over aligned groups of W lanes (W a power of two <= 64).
template <int W>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int m = W / 2; m >= 1; m >>= 1) x += __shfl_xor(x, m, W);
  return x;
}

constexpr int kThreads = 256;

template <int D, typename TIn, typename TOut>
__global__ __launch_bounds__(kThreads) void decode_kernel(float* __restrict__ state,
                                                          const TIn* __restrict__ q,
                                                          const TIn* __restrict__ k,
                                                          const TIn* __restrict__ v,
                                                          const TIn* __restrict__ beta,
                                                          const TIn* __restrict__ log_alpha,
                                                          TOut* __restrict__ o, int64_t n_states) {
  constexpr int LPR = D / 4;              // lanes per row (one float4 each)
  constexpr int RG = 8;                   // row groups per state
  constexpr int TPS = LPR * RG;           // lanes per state = 2D
  constexpr int SPB = kThreads / TPS;     // states per workgroup
  constexpr int RPT = D / RG;             // rows per lane
  static_assert(D % 32 == 0 || D == 16, "D must be 16, 32, 64 or 128");
  static_assert(SPB >= 1 && kThreads % TPS == 0, "bad decode tiling");

  const int tid = threadIdx.x;
  const int64_t s = static_cast<int64_t>(blockIdx.x) * SPB + tid / TPS;
  if (s >= n_states) return;  // whole lane groups drop out together
  const int lt = tid % TPS;
  const int c4 = lt % LPR;
  const int rg = lt / LPR;

  float4* S = reinterpret_cast<float4*>(state + s * D * D);
  float4 st[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) st[i] = S[(rg + RG * i) * LPR + c4];

  float kk[4], qq[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    kk[j] = ld_in(k, s * D + 4 * c4 + j);
    qq[j] = ld_in(q, s * D + 4 * c4 + j);
  }
  const float b = ld_in(beta, s);
  const float a = __expf(ld_in(log_alpha, s));

  float r[RPT], p[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    r[i] = st[i].x * kk[0] + st[i].y * kk[1] + st[i].z * kk[2] + st[i].w * kk[3];
    p[i] = st[i].x * qq[0] + st[i].y * qq[1] + st[i].z * qq[2] + st[i].w * qq[3];
  }
  float kq = kk[0] * qq[0] + kk[1] * qq[1] + kk[2] * qq[2] + kk[3] * qq[3];
  kq = group_sum<LPR>(kq);
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    r[i] = group_sum<LPR>(r[i]);
    p[i] = group_sum<LPR>(p[i]);
  }

#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int row = rg + RG * i;
    const float u = b * (ld_in(v, s * D + row) - a * r[i]);
    float4 x = st[i];
    x.x = a * x.x + u * kk[0];
    x.y = a * x.y + u * kk[1];
    x.z = a * x.z + u * kk[2];
    x.w = a * x.w + u * kk[3];
    S[row * LPR + c4] = x;
    if (c4 == 0) st_out(o, s * D + row, a * p[i] + u * kq);
  }
}

template <int D, typename TIn, typename TOut>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
  constexpr int SPB = kThreads / (2 * D);
  const int64_t n = a.N * a.H;
  const int64_t blocks = (n + SPB - 1) / SPB;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((decode_kernel<D, TIn, TOut>), dim3(static_cast<unsigned>(blocks)),
                     dim3(kThreads), 0, stream, a.state, static_cast<const TIn*>(a.q),
                     static_cast<const TIn*>(a.k), static_cast<const TIn*>(a.v),
                     static_cast<const TIn*>(a.beta), static_cast<const TIn*>(a.log_alpha),
                     static_cast<TOut*>(a.o), n);
  return hipGetLastError();
}

template <int D>
hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t s) {
  if (a.in_dtype == GDN_BF16) {
    return a.out_dtype == GDN_BF16 ? launch_decode_t<D, __hip_bfloat16, __hip_bfloat16>(a, s)
                                   : launch_decode_t<D, __hip_bfloat16, float>(a, s);
  }
  return a.out_dtype == GDN_BF16 ? launch_decode_t<D, float, __hip_bfloat16>(a, s)
                                 : launch_decode_t<D, float, float>(a, s);
}

}  // namespace

bool decode_supported(const DecodeArgs& a) {
  return a.D == 16 || a.D == 32 || a.D == 64 || a.D == 128;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  switch (a.D) {
    case 16: return launch_decode_d<16>(a, s);
    case 32: return launch_decode_d<32>(a, s);
    case 64: return launch_decode_d<64>(a, s);
    case 128: return launch_decode_d<128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gdn
