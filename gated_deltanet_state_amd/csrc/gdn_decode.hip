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
// accesses).  The 2 x (D/8) row dot products of a lane are reduced across the D/4 lanes of
// its row group by one butterfly reduce-scatter (D/4 - 1 exchanges, DPP and ds_swizzle, no
// LDS memory traffic) that leaves one finished dot product per lane; the per-row corrections
// are then broadcast back through a small LDS line private to the wavefront.  All loads of
// the state are issued before any reduction, so the whole 64 KiB state of a workgroup is in
// flight at once.
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

// Exchange with lane ^ M inside aligned groups of 32 lanes: DPP quad permutes for M = 1, 2
// (no LDS traffic), ds_swizzle bit-mask mode otherwise.
template <int M>
__device__ __forceinline__ float xor_lane(float x) {
  const int v = __float_as_int(x);
  if constexpr (M == 1) return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0xB1, 0xf, 0xf, false));  // [1,0,3,2]
  else if constexpr (M == 2) return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0x4E, 0xf, 0xf, false));  // [2,3,0,1]
  else return __int_as_float(__builtin_amdgcn_ds_swizzle(v, (M << 10) | 0x1f));
}

// Sum over aligned groups of W lanes (W a power of two <= 32); every lane gets the sum.
template <int W>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (W >= 32) x += xor_lane<16>(x);
  if constexpr (W >= 16) x += xor_lane<8>(x);
  if constexpr (W >= 8) x += xor_lane<4>(x);
  if constexpr (W >= 4) x += xor_lane<2>(x);
  if constexpr (W >= 2) x += xor_lane<1>(x);
  return x;
}

// Butterfly reduce-scatter of N values over aligned groups of N lanes: on return vals[0] of
// lane j (j = lane mod N) holds the group sum of value j.  At the step with partner lane ^ M
// each lane keeps the half of its 2M values selected by its bit M and receives the other half
// from its partner: N - 1 exchanges in all instead of N log2 N for N separate reductions.
template <int M>
__device__ __forceinline__ void scatter_step(float* vals, int lane) {
  const bool upper = (lane & M) != 0;
#pragma unroll
  for (int i = 0; i < M; ++i) {
    const float send = upper ? vals[i] : vals[M + i];
    const float keep = upper ? vals[M + i] : vals[i];
    vals[i] = keep + xor_lane<M>(send);
  }
}
template <int N>
__device__ __forceinline__ void reduce_scatter(float* vals, int lane) {
  if constexpr (N >= 32) scatter_step<16>(vals, lane);
  if constexpr (N >= 16) scatter_step<8>(vals, lane);
  if constexpr (N >= 8) scatter_step<4>(vals, lane);
  if constexpr (N >= 4) scatter_step<2>(vals, lane);
  if constexpr (N >= 2) scatter_step<1>(vals, lane);
}

constexpr int kThreads = 256;
typedef float f4v __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// The state rows one lane touches: float4 number lane_f4 + off of the state.  When a state's
// lanes fill whole wavefronts the base is the same in every lane, so the rows go through a
// buffer descriptor: one lane offset in a register, each row's offset a scalar constant,
// instead of one 64-bit address per row.  Loads are ordinary; stores are non-temporal (the
// descriptor's nt cache-policy bit).
template <int D, bool UNIFORM>
struct StateRows;
template <int D>
struct StateRows<D, true> {
  __amdgpu_buffer_rsrc_t r;
  int voff;
  __device__ __forceinline__ StateRows(float* base, int lane_f4) : voff(16 * lane_f4) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    const uint64_t u = static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(b)))) |
                       static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(b >> 32)))) << 32;
    r = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(u), 0, D * D * 4, 0x00020000);
  }
  __device__ __forceinline__ f4v load(int off) const {
    return __builtin_bit_cast(f4v, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 16 * off, 0));
  }
  // the store takes its row offset in the lane offset and a zero scalar offset: a store of
  // more than 8 bytes with a register scalar offset is exempt from the compiler's wait state
  // before its data registers are overwritten
  __device__ __forceinline__ void store(int off, f4v x) const {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, x), r, voff + 16 * off, 0, 2);
  }
};
template <int D>
struct StateRows<D, false> {
  f4v* p;
  __device__ __forceinline__ StateRows(float* base, int lane_f4) : p(reinterpret_cast<f4v*>(base) + lane_f4) {}
  __device__ __forceinline__ f4v load(int off) const { return p[off]; }
  __device__ __forceinline__ void store(int off, f4v x) const { __builtin_nontemporal_store(x, p + off); }
};

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
  constexpr int RPT = D / RG;             // rows per lane; 2 RPT == LPR partial sums to reduce
  static_assert(D == 16 || D == 32 || D == 64 || D == 128, "D must be 16, 32, 64 or 128");
  static_assert(2 * RPT == LPR, "one reduced value per lane");
  __shared__ float ush[SPB][D];           // per-row corrections, broadcast inside a lane group

  const int tid = threadIdx.x;
  const int slot = tid / TPS;
  const int64_t s = static_cast<int64_t>(blockIdx.x) * SPB + slot;
  if (s >= n_states) return;  // whole lane groups drop out together
  const int lt = tid % TPS;
  const int c4 = lt % LPR;                // column quad, and the lane's index inside its row group
  const int rg = lt / LPR;

  // the states stream through once per step. Ordinary loads (the non-temporal hint on the
  // loads measured about 12% slower for the same bytes); the stores stay non-temporal (plain
  // stores measured about 25% slower)
  // (the descriptor form of the serving kernel below lifts this kernel to 5 waves per SIMD
  // but measured the same, so it keeps one address per row)
  StateRows<D, false> S(state + s * D * D, rg * LPR + c4);
  f4v st[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) st[i] = S.load(i * RG * LPR);

  float kk[4], qq[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    kk[j] = ld_in(k, s * D + 4 * c4 + j);
    qq[j] = ld_in(q, s * D + 4 * c4 + j);
  }
  const float b = ld_in(beta, s);
  const float a = __expf(ld_in(log_alpha, s));

  // partial dot products: value 2i = s_row(i) . k, value 2i + 1 = s_row(i) . q
  float vals[2 * RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    vals[2 * i] = st[i][0] * kk[0] + st[i][1] * kk[1] + st[i][2] * kk[2] + st[i][3] * kk[3];
    vals[2 * i + 1] = st[i][0] * qq[0] + st[i][1] * qq[1] + st[i][2] * qq[2] + st[i][3] * qq[3];
  }
  const float kq = group_sum<LPR>(kk[0] * qq[0] + kk[1] * qq[1] + kk[2] * qq[2] + kk[3] * qq[3]);
  reduce_scatter<LPR>(vals, c4);

  // lane c4 of the group now holds r (c4 even) or p (c4 odd) of row rg + RG * (c4 / 2)
  const int row = rg + RG * (c4 >> 1);
  const float r_or_p = vals[0];
  const float u = b * (ld_in(v, s * D + row) - a * r_or_p);        // meaningful on even lanes
  const float u_even = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(u), 0xA0, 0xf, 0xf, false));  // [0,0,2,2]
  if (c4 & 1) st_out(o, s * D + row, a * r_or_p + u_even * kq);
  else ush[slot][row] = u;
  // the rows of this lane group were written by lanes of the same wavefront
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const float ui = ush[slot][rg + RG * i];
    f4v x = st[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = a * x[j] + ui * kk[j];
    S.store(i * RG * LPR, x);
  }
}

// ------------------------------------------------------------------------------------------
// Serving-side decode: a window of T tokens per sequence on states addressed through a slot
// table, with value heads sharing query/key heads, optionally with the q/k normalisation and
// the gate activations of the layer fused in, and either applying the first n_commit tokens
// to the state (commit) or leaving it untouched (verification of draft tokens).
//   * A sequence whose slot is negative or past the pool is skipped (no output written).
//   * Value head h reads query/key head h / (H / Hqk).
//   * Normalisation: x / sqrt(sum x^2 + 1e-6) over the head dimension ("Attention, Part 4",
//     a Gated DeltaNet layer normalises queries and keys to length 1).
//   * Gate activations ("Attention, Part 4", section "Where alpha and beta come from"):
//     beta = sigmoid(b), log alpha = -exp(A_log[h]) softplus(a + dt_bias[h]).
//   * KDA scales key channel j of the state by alpha_j before the step ("From Traditional
//     Attention to hybrid ones", section 7); the step is then the scalar one with alpha = 1.
// The state is read once and, on commit, written once: the tokens of the window run on the
// registers, each with the reductions of the single-step kernel above.  The state after the
// last committed token is stored as soon as it exists.  Without outputs (OUT false: commit
// alone) only the key products S k are formed and reduced.
template <int D, typename TIn, typename TOut, bool KDA, bool OUT>
__global__ __launch_bounds__(kThreads, 4) void decode_ex_kernel(DecodeExArgs a) {
  constexpr int LPR = D / 4, RG = 8, TPS = LPR * RG, SPB = kThreads / TPS, RPT = D / RG;
  static_assert(2 * RPT == LPR, "one reduced value per lane");
  __shared__ float ush[SPB][D];

  const TIn* __restrict__ q = static_cast<const TIn*>(a.q);
  const TIn* __restrict__ k = static_cast<const TIn*>(a.k);
  const TIn* __restrict__ v = static_cast<const TIn*>(a.v);
  const TIn* __restrict__ beta = static_cast<const TIn*>(a.beta);
  const TIn* __restrict__ log_alpha = static_cast<const TIn*>(a.log_alpha);
  TOut* __restrict__ o = static_cast<TOut*>(a.o);

  const int tid = threadIdx.x;
  const int lane_slot = tid / TPS;
  const int64_t s = static_cast<int64_t>(blockIdx.x) * SPB + lane_slot;  // (sequence, value head)
  if (s >= a.N * a.H) return;  // whole lane groups drop out together
  const int64_t n = s / a.H, h = s - n * a.H, hq = h / (a.H / a.Hqk);
  const int64_t row_slot = a.slots ? static_cast<int64_t>(a.slots[n]) : n;
  if (row_slot < 0 || row_slot >= a.P) return;
  int ncommit = 0;
  if (a.write_state) {
    ncommit = a.n_commit ? a.n_commit[n] : static_cast<int>(a.T);
    ncommit = ncommit < 0 ? 0 : (ncommit > a.T ? static_cast<int>(a.T) : ncommit);
  }
  const int tend = OUT ? static_cast<int>(a.T) : ncommit;
  if (tend == 0) return;

  const int lt = tid % TPS, c4 = lt % LPR, rg = lt / LPR;
  StateRows<D, (TPS >= 64)> S(a.pool + (row_slot * a.H + h) * D * D, rg * LPR + c4);
  f4v st[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) st[i] = S.load(i * RG * LPR);
  float A = 0.f, dtb = 0.f;
  if (!KDA && a.raw_gates) {
    A = __expf(a.A_log[h]);
    dtb = a.dt_bias[h];
  }

  // Commit (no outputs) keeps the state as S = cs S' with a running scale cs, the product of
  // the scalar decays so far: a token adds (u / cs) k^T to S' with one FMA per element, and
  // S' is multiplied by cs once, when stored.  If cs would fall below 2^-60 it is first
  // folded into the rows and that token takes the direct update, so 1 / cs stays finite.
  // (KDA has no scalar decay here, so cs stays 1.)
  float cs = 1.f;
  for (int t = 0; t < tend; ++t) {
    const int64_t tok = n * a.T + t;
    const int64_t qk0 = (tok * a.Hqk + hq) * D, g0 = tok * a.H + h;
    float kk[4], qq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      kk[j] = ld_in(k, qk0 + 4 * c4 + j);
      if constexpr (OUT) qq[j] = ld_in(q, qk0 + 4 * c4 + j);
    }
    if (a.qk_l2norm) {
      const float nk = group_sum<LPR>(kk[0] * kk[0] + kk[1] * kk[1] + kk[2] * kk[2] + kk[3] * kk[3]);
      const float rk = 1.f / sqrtf(nk + 1e-6f);
#pragma unroll
      for (int j = 0; j < 4; ++j) kk[j] *= rk;
      if constexpr (OUT) {
        const float nq = group_sum<LPR>(qq[0] * qq[0] + qq[1] * qq[1] + qq[2] * qq[2] + qq[3] * qq[3]);
        const float rq = 1.f / sqrtf(nq + 1e-6f);
#pragma unroll
        for (int j = 0; j < 4; ++j) qq[j] *= rq;
      }
    }
    float b = ld_in(beta, g0), dec = 1.f;
    if constexpr (KDA) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float al = expf(ld_in(log_alpha, g0 * D + 4 * c4 + j));
#pragma unroll
        for (int i = 0; i < RPT; ++i) st[i][j] *= al;
      }
    } else {
      float g = ld_in(log_alpha, g0);
      if (a.raw_gates) {
        b = 1.f / (1.f + expf(-b));
        const float x = g + dtb;
        g = -A * (fmaxf(x, 0.f) + log1pf(expf(-fabsf(x))));  // softplus, no overflow
      }
      dec = expf(g);
    }
    bool lazy = false;
    float rc = 1.f;
    if constexpr (!OUT) {
      const float cn = cs * dec;
      lazy = cn >= 0x1p-60f;
      if (lazy) {
        rc = 1.f / cn;
        cs = cn;
      } else {
#pragma unroll
        for (int i = 0; i < RPT; ++i) st[i] *= cs;
        cs = 1.f;
      }
    }

    if constexpr (OUT) {
      float vals[2 * RPT];
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        vals[2 * i] = st[i][0] * kk[0] + st[i][1] * kk[1] + st[i][2] * kk[2] + st[i][3] * kk[3];
        vals[2 * i + 1] = st[i][0] * qq[0] + st[i][1] * qq[1] + st[i][2] * qq[2] + st[i][3] * qq[3];
      }
      const float kq = group_sum<LPR>(kk[0] * qq[0] + kk[1] * qq[1] + kk[2] * qq[2] + kk[3] * qq[3]);
      reduce_scatter<LPR>(vals, c4);
      const int row = rg + RG * (c4 >> 1);
      const float r_or_p = vals[0];
      const float u = b * (ld_in(v, (tok * a.H + h) * D + row) - dec * r_or_p);
      const float u_even = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(u), 0xA0, 0xf, 0xf, false));
      if (c4 & 1) {
        st_out(o, (tok * a.H + h) * D + row, dec * r_or_p + u_even * kq);
      } else {
        ush[lane_slot][row] = u;
      }
    } else {
      // RPT key products over the row's LPR = 2 RPT lanes: reduce-scatter inside each half,
      // then add the other half's partial sums; lanes c4 and c4 + RPT hold row value c4 mod RPT
      float vals[RPT];
#pragma unroll
      for (int i = 0; i < RPT; ++i)
        vals[i] = st[i][0] * kk[0] + st[i][1] * kk[1] + st[i][2] * kk[2] + st[i][3] * kk[3];
      reduce_scatter<RPT>(vals, c4);
      const float r = vals[0] + xor_lane<RPT>(vals[0]);
      const int row = rg + RG * (c4 & (RPT - 1));
      // lazy: r is S'_{t-1} k and the stored correction is u / cs = beta (v / cs - r)
      const float vr = ld_in(v, (tok * a.H + h) * D + row);
      if (c4 < RPT) ush[lane_slot][row] = lazy ? b * (vr * rc - r) : b * (vr - dec * r);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (lazy) {
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const float ui = ush[lane_slot][rg + RG * i];
#pragma unroll
        for (int j = 0; j < 4; ++j) st[i][j] += ui * kk[j];
      }
    } else {
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const float ui = ush[lane_slot][rg + RG * i];
#pragma unroll
        for (int j = 0; j < 4; ++j) st[i][j] = dec * st[i][j] + ui * kk[j];
      }
    }
    // the next token overwrites the corrections only after every lane has read them
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (t + 1 == ncommit) {
#pragma unroll
      for (int i = 0; i < RPT; ++i) S.store(i * RG * LPR, OUT ? st[i] : st[i] * cs);
    }
  }
}


// Commit of accepted tokens (the state is written, no outputs) at d = 128, where one state
// fills the workgroup.  The arithmetic is that of decode_ex_kernel without outputs, token for
// token, so the two give the same bits; what differs is where the per-token inputs come from.
// The window's keys (normalised when asked), values and gates, at most kCommitStage tokens,
// are staged in LDS by one half-wavefront per token, with the loads issued before the
// state's: the token loop then reads them from LDS and no token waits for a global load of
// its own.  Longer windows run on decode_ex_kernel.
constexpr int kCommitStage = 8;
template <typename TIn, bool KDA>
__global__ __launch_bounds__(kThreads, 4) void decode_commit128_kernel(DecodeExArgs a) {
  constexpr int D = 128, LPR = D / 4, RG = 8, RPT = D / RG, W = kCommitStage;
  static_assert(LPR * RG == kThreads && W * LPR == kThreads, "one state per workgroup, one token per half-wave");
  __shared__ float ush[D];
  __shared__ f4v kw[W][LPR];                  // keys, normalised when asked
  __shared__ float vw[W][D];                  // values
  __shared__ float bw[W], dw[W];              // beta and the scalar decay
  __shared__ f4v aw[KDA ? W : 1][LPR];        // per-channel decays (KDA)

  const TIn* __restrict__ k = static_cast<const TIn*>(a.k);
  const TIn* __restrict__ v = static_cast<const TIn*>(a.v);
  const TIn* __restrict__ beta = static_cast<const TIn*>(a.beta);
  const TIn* __restrict__ log_alpha = static_cast<const TIn*>(a.log_alpha);

  const int tid = threadIdx.x;
  const int64_t s = blockIdx.x;  // (sequence, value head); the whole workgroup drops out together
  if (s >= a.N * a.H) return;
  const int64_t n = s / a.H, h = s - n * a.H, hq = h / (a.H / a.Hqk);
  const int64_t row_slot = a.slots ? static_cast<int64_t>(a.slots[n]) : n;
  if (row_slot < 0 || row_slot >= a.P) return;
  int ncommit = a.n_commit ? a.n_commit[n] : static_cast<int>(a.T);
  ncommit = ncommit < 0 ? 0 : (ncommit > a.T ? static_cast<int>(a.T) : ncommit);
  if (ncommit == 0) return;

  const int c4 = tid % LPR, rg = tid / LPR;   // as in decode_ex_kernel: rg is the half-wave
  float A = 0.f, dtb = 0.f;
  if (!KDA && a.raw_gates) {
    A = __expf(a.A_log[h]);
    dtb = a.dt_bias[h];
  }
  // staging: half-wave w takes token w, lane c4 its columns 4 c4 .. 4 c4 + 3
  if (rg < ncommit) {
    const int w = rg;
    const int64_t tok = n * a.T + w;
    const int64_t qk0 = (tok * a.Hqk + hq) * D, g0 = tok * a.H + h;
    float kk[4], vv[4], al[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      kk[j] = ld_in(k, qk0 + 4 * c4 + j);
      vv[j] = ld_in(v, g0 * D + 4 * c4 + j);
      if constexpr (KDA) al[j] = ld_in(log_alpha, g0 * D + 4 * c4 + j);
    }
    float b = ld_in(beta, g0), g = 0.f;
    if constexpr (!KDA) g = ld_in(log_alpha, g0);
    if (a.qk_l2norm) {
      const float nk = group_sum<LPR>(kk[0] * kk[0] + kk[1] * kk[1] + kk[2] * kk[2] + kk[3] * kk[3]);
      const float rk = 1.f / sqrtf(nk + 1e-6f);
#pragma unroll
      for (int j = 0; j < 4; ++j) kk[j] *= rk;
    }
    kw[w][c4] = f4v{kk[0], kk[1], kk[2], kk[3]};
    *reinterpret_cast<f4v*>(&vw[w][4 * c4]) = f4v{vv[0], vv[1], vv[2], vv[3]};
    if constexpr (KDA) aw[w][c4] = f4v{expf(al[0]), expf(al[1]), expf(al[2]), expf(al[3])};
    if (c4 == 0) {
      float dec = 1.f;
      if constexpr (!KDA) {
        if (a.raw_gates) {
          b = 1.f / (1.f + expf(-b));
          const float x = g + dtb;
          g = -A * (fmaxf(x, 0.f) + log1pf(expf(-fabsf(x))));  // softplus, no overflow
        }
        dec = expf(g);
      }
      bw[w] = b;
      dw[w] = dec;
    }
  }
  StateRows<D, true> S(a.pool + (row_slot * a.H + h) * D * D, rg * LPR + c4);
  f4v st[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) st[i] = S.load(i * RG * LPR);
  __syncthreads();

  // The state is kept as cs S' with a running scale cs, the product of the decays so far: a
  // token adds (u / cs) k^T to S' with one FMA per element.  A token whose decay would take cs
  // below 2^-60 first multiplies cs and its own decay into the rows (any decay, 0 included)
  // and continues from cs = 1, so 1 / cs stays finite.
  float cs = 1.f;
#pragma unroll 1
  for (int t = 0; t < ncommit; ++t) {
    const f4v kv = kw[t][c4];
    const float kk[4] = {kv[0], kv[1], kv[2], kv[3]};
    // the gates are the same in every lane: scalar registers, so the branch below is uniform
    const float b = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(bw[t])));
    const float dec = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(dw[t])));
    if constexpr (KDA) {
      const f4v al = aw[t][c4];
#pragma unroll
      for (int i = 0; i < RPT; ++i) st[i] *= al;
    }
    const float cn = cs * dec;
    float rc;
    if (cn >= 0x1p-60f) {
      cs = cn;
      rc = 1.f / cn;
    } else {
#pragma unroll
      for (int i = 0; i < RPT; ++i) st[i] = (st[i] * cs) * dec;
      cs = 1.f;
      rc = 1.f;
    }
    float vals[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i)
      vals[i] = st[i][0] * kk[0] + st[i][1] * kk[1] + st[i][2] * kk[2] + st[i][3] * kk[3];
    reduce_scatter<RPT>(vals, c4);
    const float r = vals[0] + xor_lane<RPT>(vals[0]);
    const int row = rg + RG * (c4 & (RPT - 1));
    // r is S'_{t-1} k and the stored correction is u / cs = beta (v / cs - r)
    if (c4 < RPT) ush[row] = b * (vw[t][row] * rc - r);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const float ui = ush[rg + RG * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) st[i][j] += ui * kk[j];
    }
    // the next token overwrites the corrections only after every lane has read them
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
#pragma unroll
  for (int i = 0; i < RPT; ++i) S.store(i * RG * LPR, st[i] * cs);
}

// ------------------------------------------------------------------------------------------
// Matrix-core form of draft-token verification (outputs only, the state is not written) for
// the scalar gate at d = 128 and windows of at most 8 tokens.  The window is one chunk of the
// chunkwise form ("Hybrid Linear Attention Architecture Design Explained", section 4), with S
// the state entering the window, k, q normalised when asked, G_t the inclusive prefix of
// log alpha and gamma_t = e^{G_t}:
//   r_t = S k_t, p_t = S q_t                          (one fp32 matrix-core product)
//   x_t = beta_t (v_t - gamma_t r_t)
//   u_t = x_t - sum_{j<t} beta_t (k_t.k_j) e^{G_t - G_j} u_j
//   o_t = gamma_t p_t + sum_{j<=t} (q_t.k_j) e^{G_t - G_j} u_j
// which is the token loop above regrouped: the state products run on v_mfma_f32_16x16x4_f32
// (full fp32), the W x W algebra per value channel on 32 lanes.  The per-token reductions of
// the loop form, which bound its instruction issue, are gone.
//
// One workgroup per (sequence, value head), four wavefronts; wave w owns value channels
// 32 w .. 32 w + 31.  Its slice of S^T is read straight into MFMA accumulator layout, one
// 16-row half n at a time (fewer live registers, more waves per SIMD): tile j of half n holds
// S^T[dk = 16 j + 4 (l/16) + i][dv = 32 w + 16 n + l%16] in component i.
// Used as the B operand of a 16x16x4 product, component i of the tile is the k-block whose
// four contraction indices are dk = 16 j + 4 kb + i, kb = l/16; the A operand (the window's
// keys and queries, one row per lane%16) is loaded with the same index pattern, so no
// transposition is ever needed.  The same A fragments, used as both operands, give the Gram
// of the window's keys and queries (their norms on its diagonal); each wave forms it over a
// quarter of the key channels and the four parts are summed through LDS.
constexpr int kWinMax = 8;
// Four consecutive inputs as fp32 (one 8- or 16-byte load), zeros when !live.
__device__ __forceinline__ void ld4(const float* p, bool live, float (&x)[4]) {
  f4v y = {0.f, 0.f, 0.f, 0.f};
  if (live) y = *reinterpret_cast<const f4v*>(p);
  x[0] = y[0]; x[1] = y[1]; x[2] = y[2]; x[3] = y[3];
}
__device__ __forceinline__ void ld4(const __hip_bfloat16* p, bool live, float (&x)[4]) {
  uint2 y = {0u, 0u};
  if (live) y = *reinterpret_cast<const uint2*>(p);
  x[0] = __uint_as_float(y.x << 16); x[1] = __uint_as_float(y.x & 0xffff0000u);
  x[2] = __uint_as_float(y.y << 16); x[3] = __uint_as_float(y.y & 0xffff0000u);
}
template <typename TIn, typename TOut>
// (fp32 inputs stage 4 KiB of values instead of 2: their LDS allows 6 workgroups per CU)
__global__ __launch_bounds__(256, sizeof(TIn) == 2 ? 8 : 6) void decode_win_mfma_kernel(DecodeExArgs a) {
  constexpr int D = 128;
  typedef float f4 __attribute__((ext_vector_type(4)));
  // The staged rows are dead once the products are done; S k_t, S q_t reuse their space (written
  // after the barrier that follows the products).
  __shared__ union {
    float ash[16][D + 8];                       // rows [k_0..k_{W-1}, q_0..q_{W-1}, 0..] (8-bank row skew)
    float rsh[4][16][33];                       // S k_t and S q_t per wave: [row][value channel]
  } lu;
  __shared__ float gpart[4][16][16];            // per wave: Gram over its quarter of the key channels
  __shared__ float gsh[4][16][16];              // Gram of the window's rows [k_0..k_{W-1}, q_0..q_{W-1}]
  __shared__ __align__(16) TIn vsh[kWinMax][D]; // the window's values, as stored
  auto& ash = lu.ash;
  auto& rsh = lu.rsh;

  const TIn* __restrict__ q = static_cast<const TIn*>(a.q);
  const TIn* __restrict__ k = static_cast<const TIn*>(a.k);
  const TIn* __restrict__ v = static_cast<const TIn*>(a.v);
  const TIn* __restrict__ beta = static_cast<const TIn*>(a.beta);
  const TIn* __restrict__ log_alpha = static_cast<const TIn*>(a.log_alpha);
  TOut* __restrict__ o = static_cast<TOut*>(a.o);

  const int64_t s = blockIdx.x;  // (sequence, value head); the grid is exactly N H
  const int64_t n = s / a.H, h = s - n * a.H, hq = h / (a.H / a.Hqk);
  const int64_t row_slot = a.slots ? static_cast<int64_t>(a.slots[n]) : n;
  if (row_slot < 0 || row_slot >= a.P) return;  // uniform over the workgroup
  const int W = static_cast<int>(a.T);

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, lr = l & 15, lg = l >> 4;

  // the first 16 rows of the state slice (the second half is loaded once these are used).
  // Ordinary loads: each 128-byte line is read as two 64-byte halves by consecutive
  // instructions, and with the non-temporal hint the line can leave the cache in between
  // and be fetched twice.
  f4* S = reinterpret_cast<f4*>(a.pool + (row_slot * a.H + h) * D * D);
  f4 St[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) St[j] = S[((32 * w + lr) * D + 16 * j + 4 * lg) / 4];

  // the window's key and query rows, staged once for the four waves: thread tid holds
  // channels 8 (tid % 16) .. + 7 of row tid / 16
  {
    const int r = tid >> 4, c = 8 * (tid & 15);
    const bool live = r < 2 * W;
    const int t = r < W ? r : (live ? r - W : 0);
    const TIn* src = (r < W ? k : q) + ((n * a.T + t) * a.Hqk + hq) * D + c;
    float x[4], y[4];
    ld4(src, live, x);
    ld4(src + 4, live, y);
    *reinterpret_cast<f4*>(&ash[r][c]) = f4{x[0], x[1], x[2], x[3]};
    *reinterpret_cast<f4*>(&ash[r][c + 4]) = f4{y[0], y[1], y[2], y[3]};
    // the value rows, copied as stored (16-byte pieces), by the threads of the key rows
    if (r < W) {
      typedef unsigned int u4 __attribute__((ext_vector_type(4)));
      const u4* vs = reinterpret_cast<const u4*>(v + ((n * a.T + r) * a.H + h) * D + c);
      u4* vd = reinterpret_cast<u4*>(&vsh[r][c]);
#pragma unroll
      for (int e = 0; e < static_cast<int>(8 * sizeof(TIn) / 16); ++e) vd[e] = vs[e];
    }
  }

  // gates of the window: lane t < W loads beta_t and log alpha_t (formed after the products)
  float gb = 0.f, gg = 0.f;
  if (l < W) {
    const int64_t g0 = (n * a.T + l) * a.H + h;
    gb = ld_in(beta, g0);
    gg = ld_in(log_alpha, g0);
  }

  // Gram of the rows, and S k_t, S q_t: contraction over the 128 key channels.  A fragment:
  // row l%16, channels 16 j + 4 (l/16) .. + 3 (one conflict-free 16-byte read per j).
  __syncthreads();  // the rows are staged
  const f4 zero = {0.f, 0.f, 0.f, 0.f};
  f4 gm = zero, rp[2] = {zero, zero};
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {  // 16-row halves of the slice, one after the other
    if (nb == 1) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        St[j] = S[((32 * w + 16 + lr) * D + 16 * j + 4 * lg) / 4];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const f4 af = *reinterpret_cast<const f4*>(&ash[lr][16 * j + 4 * lg]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (nb == 0 && j >> 1 == w) gm = __builtin_amdgcn_mfma_f32_16x16x4f32(af[i], af[i], gm, 0, 0, 0);  // uniform
        rp[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[i], St[j][i], rp[nb], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) gpart[w][4 * lg + e][lr] = gm[e];
  __syncthreads();  // the four parts of the Gram; every wave is done with the staged rows
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int r = 4 * lg + e;
    gsh[w][r][lr] = (gpart[0][r][lr] + gpart[1][r][lr]) + (gpart[2][r][lr] + gpart[3][r][lr]);
    rsh[w][r][lr] = rp[0][e];
    rsh[w][r][16 + lr] = rp[1][e];
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // gates: lane t < W forms beta_t and log alpha_t, every lane then reads them
  float G[kWinMax], bt[kWinMax];
  {
    if (a.raw_gates && l < W) {
      gb = __builtin_amdgcn_rcpf(1.f + __expf(-gb));
      const float x = gg + a.dt_bias[h];
      gg = -__expf(a.A_log[h]) * (fmaxf(x, 0.f) + log1pf(__expf(-fabsf(x))));  // softplus, no overflow
    }
    float run = 0.f;
#pragma unroll
    for (int t = 0; t < kWinMax; ++t) {
      run += __shfl(gg, t, 64);
      G[t] = run;
      bt[t] = __shfl(gb, t, 64);
    }
  }

  // normalisation factors 1 / |k_t|, 1 / |q_t| (the Gram's diagonal), every lane
  float rk[kWinMax], rq[kWinMax];
#pragma unroll
  for (int t = 0; t < kWinMax; ++t) {
    rk[t] = 1.f;
    rq[t] = 1.f;
    if (a.qk_l2norm && t < W) {
      rk[t] = __builtin_amdgcn_rsqf(gsh[w][t][t] + 1e-6f);
      rq[t] = __builtin_amdgcn_rsqf(gsh[w][W + t][W + t] + 1e-6f);
    }
  }

  // per value channel: the substitution and the outputs (lanes 0..31)
  if (l < 32) {
    const int dv = 32 * w + l;
    float u[kWinMax];
#pragma unroll
    for (int t = 0; t < kWinMax; ++t) {
      u[t] = 0.f;
      if (t >= W) continue;  // uniform
      const int64_t tok = n * a.T + t;
      const float gam = __expf(G[t]);
      float x = bt[t] * (ld_in(&vsh[t][0], dv) - gam * rk[t] * rsh[w][t][l]);
      float dq[kWinMax];  // e^{G_t - G_j} / |k_j|, j <= t
#pragma unroll
      for (int j = 0; j <= t; ++j) dq[j] = __expf(G[t] - G[j]) * rk[j];
      const float ct = bt[t] * rk[t];
#pragma unroll
      for (int j = 0; j < t; ++j) x -= ct * gsh[w][t][j] * dq[j] * u[j];
      u[t] = x;
      float y = 0.f;
#pragma unroll
      for (int j = 0; j <= t; ++j) y += gsh[w][W + t][j] * dq[j] * u[j];
      st_out(o, (tok * a.H + h) * D + dv, rq[t] * (gam * rsh[w][W + t][l] + y));
    }
  }
}

template <int D, typename TIn, typename TOut>
hipError_t launch_decode_ex_t(const DecodeExArgs& a, hipStream_t stream) {
  constexpr int SPB = kThreads / (2 * D);
  const int64_t units = a.N * a.H;
  const int64_t blocks = (units + SPB - 1) / SPB;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if constexpr (D == 128) {
    // Verification windows (outputs only) take the matrix-core form.  A window that writes the
    // state stays on the row-coalesced kernel: reading and writing every state is HBM-bound
    // there already, and the accumulator layout moves the state in 64-byte pieces per row.
    // its key/query loads move 4 elements at once and its value copies 16 bytes: the bases
    // must be aligned to that
    const uintptr_t qk_align = 4 * sizeof(TIn);
    const bool qk_aligned = (reinterpret_cast<uintptr_t>(a.q) | reinterpret_cast<uintptr_t>(a.k)) % qk_align == 0 &&
                            reinterpret_cast<uintptr_t>(a.v) % 16 == 0;
    if (!a.kda && !a.write_state && a.o && a.T <= kWinMax && qk_aligned && units <= 0x7fffffff) {
      hipLaunchKernelGGL((decode_win_mfma_kernel<TIn, TOut>), dim3(static_cast<unsigned>(units)), dim3(256), 0,
                         stream, a);
      return hipGetLastError();
    }
  }
  const dim3 grid(static_cast<unsigned>(blocks));
  if constexpr (D == 128) {
    if (a.write_state && !a.o && a.T <= kCommitStage) {
      if (a.kda) hipLaunchKernelGGL((decode_commit128_kernel<TIn, true>), grid, dim3(kThreads), 0, stream, a);
      else hipLaunchKernelGGL((decode_commit128_kernel<TIn, false>), grid, dim3(kThreads), 0, stream, a);
      return hipGetLastError();
    }
  }
  if (a.kda) {
    if (a.o) hipLaunchKernelGGL((decode_ex_kernel<D, TIn, TOut, true, true>), grid, dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL((decode_ex_kernel<D, TIn, TOut, true, false>), grid, dim3(kThreads), 0, stream, a);
  } else {
    if (a.o) hipLaunchKernelGGL((decode_ex_kernel<D, TIn, TOut, false, true>), grid, dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL((decode_ex_kernel<D, TIn, TOut, false, false>), grid, dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_decode_ex_d(const DecodeExArgs& a, hipStream_t s) {
  if (a.in_dtype == GDN_BF16) {
    return a.out_dtype == GDN_BF16 ? launch_decode_ex_t<D, __hip_bfloat16, __hip_bfloat16>(a, s)
                                   : launch_decode_ex_t<D, __hip_bfloat16, float>(a, s);
  }
  return a.out_dtype == GDN_BF16 ? launch_decode_ex_t<D, float, __hip_bfloat16>(a, s)
                                 : launch_decode_ex_t<D, float, float>(a, s);
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

hipError_t launch_decode_ex(const DecodeExArgs& a, hipStream_t s) {
  switch (a.D) {
    case 16: return launch_decode_ex_d<16>(a, s);
    case 32: return launch_decode_ex_d<32>(a, s);
    case 64: return launch_decode_ex_d<64>(a, s);
    case 128: return launch_decode_ex_d<128>(a, s);
    default: return hipErrorInvalidValue;
  }
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
