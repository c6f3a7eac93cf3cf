// gdn_chunk_valu.hip -- chunkwise prefill of the gated delta rule (GDN) and of KDA in
// plain fp32 on the vector units (gfx950).  This is the precise path: fp32 inputs, small
// head sizes, and any (D, chunk) the matrix-core kernel does not take.
//
// Chunkwise form ("Hybrid Linear Attention Architecture Design Explained", section 4:
// cross-chunk state update and intra-chunk output; "Hybrid attention", section "Training
// a recurrence in parallel": a small lower-triangular system inside a chunk, only the
// state between chunks), written in the d_v x d_k state convention.  Per chunk of n <= C
// tokens with state S on entry, G_r = sum_{s<=r} log alpha_s (per key channel for KDA):
//   A = strict_tril(diag(beta) ((K*e^G) (K*e^-G)^T))     decay-weighted key Gram
//   T = (I + A)^-1                                        unit lower triangular
//   X = diag(beta) (V - (K*e^G) S^T),   U = T X           corrected values
//   O = (Q*e^G) S^T + tril((Q*e^G)(K*e^-G)^T) U            outputs (inclusive mask)
//   S <- S Diag(e^{G_n}) + U^T (K * e^{G_n - G})           hand-off to the next chunk
// where the decay products e^{G_r - G_j} (j <= r) are formed directly per term, so no
// factor ever exceeds 1.  A ragged tail is padded with identity steps (q = k = v = 0,
// beta = 0, log alpha = 0), which change nothing ("Attention, Part 4", section 6).
//
// One workgroup owns one (batch, head) stream and DVT of its D value rows; the state tile
// lives in LDS for the whole sequence.
#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>

#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kCmax = 64;

__device__ __forceinline__ float ld_in(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ld_in(const __hip_bfloat16* p, int64_t i) {
  const uint16_t b = reinterpret_cast<const uint16_t*>(p)[i];
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ void st_out(float* p, int64_t i, float x) { p[i] = x; }
__device__ __forceinline__ void st_out(__hip_bfloat16* p, int64_t i, float x) {
  p[i] = __float2bfloat16(x);
}

template <int D, bool KDA>
struct ValuSmem {
  static constexpr int DVT = D < 16 ? D : 16;  // value rows per workgroup
  static constexpr int GD = KDA ? D : 1;        // decay channels
  float q[kCmax][D + 1];
  float k[kCmax][D + 1];
  float v[kCmax][DVT];
  float beta[kCmax];
  float g[kCmax][GD];     // log alpha, then its inclusive prefix sum G
  float s[DVT][D + 1];    // state tile: value rows [c0, c0 + DVT), all key channels
  float a[kCmax][kCmax + 1];   // A, later reused for the causal score matrix P
  float t[kCmax][kCmax + 1];   // T = (I + A)^-1
  float x[kCmax][DVT];
  float u[kCmax][DVT];
};

template <int D, bool KDA, typename TIn, typename TOut>
__global__ __launch_bounds__(kThreads) void chunk_valu_kernel(ChunkArgs p) {
  using Sm = ValuSmem<D, KDA>;
  constexpr int DVT = Sm::DVT;
  constexpr int NT = D / DVT;
  static_assert(sizeof(Sm) <= 160 * 1024, "LDS budget");
  __shared__ Sm sm;

  const TIn* __restrict__ Q = static_cast<const TIn*>(p.q);
  const TIn* __restrict__ K = static_cast<const TIn*>(p.k);
  const TIn* __restrict__ V = static_cast<const TIn*>(p.v);
  const TIn* __restrict__ Bt = static_cast<const TIn*>(p.beta);
  const TIn* __restrict__ LA = static_cast<const TIn*>(p.log_alpha);
  TOut* __restrict__ O = static_cast<TOut*>(p.o);

  const int tid = threadIdx.x;
  const int tile = blockIdx.x % NT;
  const int64_t bh = blockIdx.x / NT;
  const int c0 = tile * DVT;
  const int C = p.chunk;
  const int64_t T = p.T;

  for (int e = tid; e < DVT * D; e += kThreads) {
    const int c = e / D, i = e % D;
    sm.s[c][i] = p.s0 ? p.s0[(bh * D + c0 + c) * D + i] : 0.f;
  }

  const int64_t nchunks = (T + C - 1) / C;
  for (int64_t ci = 0; ci < nchunks; ++ci) {
    const int64_t t0 = ci * C;
    const int n = static_cast<int>(T - t0 < C ? T - t0 : C);
    __syncthreads();  // previous chunk's readers of q/k/v/g/s are done
    for (int e = tid; e < C * D; e += kThreads) {
      const int r = e / D, i = e % D;
      const bool in = r < n;
      const int64_t off = ((bh * T) + t0 + r) * D + i;
      sm.q[r][i] = in ? ld_in(Q, off) : 0.f;
      sm.k[r][i] = in ? ld_in(K, off) : 0.f;
      if (KDA) sm.g[r][i % Sm::GD] = in ? ld_in(LA, off) : 0.f;
    }
    for (int e = tid; e < C * DVT; e += kThreads) {
      const int r = e / DVT, c = e % DVT;
      sm.v[r][c] = r < n ? ld_in(V, ((bh * T) + t0 + r) * D + c0 + c) : 0.f;
    }
    for (int r = tid; r < C; r += kThreads) {
      sm.beta[r] = r < n ? ld_in(Bt, bh * T + t0 + r) : 0.f;
      if (!KDA) sm.g[r][0] = r < n ? ld_in(LA, bh * T + t0 + r) : 0.f;
    }
    __syncthreads();
    // inclusive prefix sum of log alpha over the chunk, per decay channel
    for (int i = tid; i < Sm::GD; i += kThreads) {
      float acc = 0.f;
      for (int r = 0; r < C; ++r) {
        acc += sm.g[r][i];
        sm.g[r][i] = acc;
      }
    }
    __syncthreads();

    // A (strictly lower) and X
    for (int e = tid; e < C * C; e += kThreads) {
      const int r = e / C, j = e % C;
      float acc = 0.f;
      if (j < r) {
        if (KDA) {
          for (int i = 0; i < D; ++i) acc += sm.k[r][i] * sm.k[j][i] * __expf(sm.g[r][i] - sm.g[j][i]);
        } else {
          for (int i = 0; i < D; ++i) acc += sm.k[r][i] * sm.k[j][i];
          acc *= __expf(sm.g[r][0] - sm.g[j][0]);
        }
        acc *= sm.beta[r];
      }
      sm.a[r][j] = acc;
    }
    for (int e = tid; e < C * DVT; e += kThreads) {
      const int r = e / DVT, c = e % DVT;
      float acc = 0.f;
      if (KDA) {
        for (int i = 0; i < D; ++i) acc += sm.k[r][i] * __expf(sm.g[r][i]) * sm.s[c][i];
      } else {
        for (int i = 0; i < D; ++i) acc += sm.k[r][i] * sm.s[c][i];
        acc *= __expf(sm.g[r][0]);
      }
      sm.x[r][c] = sm.beta[r] * (sm.v[r][c] - acc);
    }
    __syncthreads();

    // T = (I + A)^-1 by forward substitution; lane n owns column n (no barriers needed:
    // each lane only reads back what it wrote itself)
    for (int nc = tid; nc < C; nc += kThreads) {
      for (int r = 0; r < C; ++r) {
        float val;
        if (r < nc) {
          val = 0.f;
        } else if (r == nc) {
          val = 1.f;
        } else {
          float acc = 0.f;
          for (int j = nc; j < r; ++j) acc += sm.a[r][j] * sm.t[j][nc];
          val = -acc;
        }
        sm.t[r][nc] = val;
      }
    }
    __syncthreads();

    // U = T X, and the causal score matrix P (inclusive) into a[][] (A is no longer needed)
    for (int e = tid; e < C * DVT; e += kThreads) {
      const int r = e / DVT, c = e % DVT;
      float acc = 0.f;
      for (int j = 0; j <= r; ++j) acc += sm.t[r][j] * sm.x[j][c];
      sm.u[r][c] = acc;
    }
    for (int e = tid; e < C * C; e += kThreads) {
      const int r = e / C, j = e % C;
      float acc = 0.f;
      if (j <= r) {
        if (KDA) {
          for (int i = 0; i < D; ++i) acc += sm.q[r][i] * sm.k[j][i] * __expf(sm.g[r][i] - sm.g[j][i]);
        } else {
          for (int i = 0; i < D; ++i) acc += sm.q[r][i] * sm.k[j][i];
          acc *= __expf(sm.g[r][0] - sm.g[j][0]);
        }
      }
      sm.a[r][j] = acc;
    }
    __syncthreads();

    // O = (Q e^G) S^T + P U
    for (int e = tid; e < n * DVT; e += kThreads) {
      const int r = e / DVT, c = e % DVT;
      float acc = 0.f;
      if (KDA) {
        for (int i = 0; i < D; ++i) acc += sm.q[r][i] * __expf(sm.g[r][i]) * sm.s[c][i];
      } else {
        for (int i = 0; i < D; ++i) acc += sm.q[r][i] * sm.s[c][i];
        acc *= __expf(sm.g[r][0]);
      }
      for (int j = 0; j <= r; ++j) acc += sm.a[r][j] * sm.u[j][c];
      st_out(O, ((bh * T) + t0 + r) * D + c0 + c, acc);
    }
    __syncthreads();

    // S <- S Diag(e^{G_last}) + U^T (K * e^{G_last - G})
    for (int e = tid; e < DVT * D; e += kThreads) {
      const int c = e / D, i = e % D;
      const int gi = KDA ? i : 0;
      const float glast = sm.g[C - 1][gi];
      float acc = sm.s[c][i] * __expf(glast);
      for (int j = 0; j < C; ++j) acc += sm.u[j][c] * sm.k[j][i] * __expf(glast - sm.g[j][gi]);
      sm.s[c][i] = acc;
    }
    __syncthreads();

    const int64_t tend = t0 + n;
    if (p.s_ckpt && n == C && tend % p.ckpt_every == 0) {
      const int64_t idx = tend / p.ckpt_every - 1;
      float* dst = p.s_ckpt + ((bh * p.n_ckpt + idx) * D + c0) * D;
      for (int e = tid; e < DVT * D; e += kThreads) dst[e] = sm.s[e / D][e % D];
    }
  }
  __syncthreads();
  if (p.s_final) {
    float* dst = p.s_final + (bh * D + c0) * D;
    for (int e = tid; e < DVT * D; e += kThreads) dst[e] = sm.s[e / D][e % D];
  }
}

template <int D, bool KDA, typename TIn, typename TOut>
hipError_t launch_t(const ChunkArgs& a, hipStream_t s) {
  constexpr int NT = D / ValuSmem<D, KDA>::DVT;
  const int64_t blocks = a.B * a.H * NT;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((chunk_valu_kernel<D, KDA, TIn, TOut>), dim3(static_cast<unsigned>(blocks)),
                     dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int D, bool KDA>
hipError_t launch_dk(const ChunkArgs& a, hipStream_t s) {
  if (a.in_dtype == GDN_BF16)
    return a.out_dtype == GDN_BF16 ? launch_t<D, KDA, __hip_bfloat16, __hip_bfloat16>(a, s)
                                   : launch_t<D, KDA, __hip_bfloat16, float>(a, s);
  return a.out_dtype == GDN_BF16 ? launch_t<D, KDA, float, __hip_bfloat16>(a, s)
                                 : launch_t<D, KDA, float, float>(a, s);
}

template <int D>
hipError_t launch_d(const ChunkArgs& a, bool kda, hipStream_t s) {
  return kda ? launch_dk<D, true>(a, s) : launch_dk<D, false>(a, s);
}

}  // namespace

bool chunk_valu_supported(const ChunkArgs& a) {
  return (a.D == 16 || a.D == 32 || a.D == 64 || a.D == 128) && a.chunk <= kCmax &&
         (a.chunk == 16 || a.chunk == 32 || a.chunk == 64);
}

hipError_t launch_chunk_valu(const ChunkArgs& a, bool kda, hipStream_t s) {
  switch (a.D) {
    case 16: return launch_d<16>(a, kda, s);
    case 32: return launch_d<32>(a, kda, s);
    case 64: return launch_d<64>(a, kda, s);
    case 128: return launch_d<128>(a, kda, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gdn
