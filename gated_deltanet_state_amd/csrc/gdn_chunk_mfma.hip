// gdn_chunk_mfma.hip -- matrix-core chunkwise prefill of the gated delta rule for gfx950
// (bf16 inputs, d_k = d_v = 128, chunk = 64, fp32 state and accumulation).
//
// Method ("Hybrid Linear Attention Architecture Design Explained", section 4: cross-chunk
// state update and intra-chunk output; "Hybrid attention", section "Training a recurrence
// in parallel": inside a chunk the writes depend on each other only through a small
// lower-triangular system, between chunks only the state is passed on).  In the
// d_v x d_k convention, for a chunk of tokens r = 0..63 entering with state S, with
// G_r = sum_{s<=r} log alpha_s, gamma_r = e^{G_r} and D_rj = e^{G_r - G_j}:
//   A = strict_tril(diag(beta) (K K^T * D))           (64 x 64)
//   X = diag(beta) (V - diag(gamma) K S^T)             (64 x d_v)
//   (I + A) U = X                                      unit lower-triangular system
//   O = diag(gamma) Q S^T + tril(Q K^T * D) U          outputs
//   S <- gamma_63 S + U^T diag(e^{G_63 - G}) K         state handed to the next chunk
//
// Work decomposition: a workgroup owns one (batch, head) stream and a 32-row slice of the
// value channels (the recurrence multiplies S only from the right, so value rows evolve
// independently); the four slices of a stream are placed on the same XCD so they share its
// L2.  The slice of S lives in MFMA accumulators (fp32) for the whole sequence.
//
// Eight wavefronts run a two-stage pipeline over the chunks.  Everything that does not
// depend on the state -- the decay-weighted Gram matrix A, the causal scores P and the
// inverses of the 16x16 diagonal blocks of (I + A) -- is produced for chunk c+1 by six
// wavefronts while two wavefronts run chunk c's state-coupled triangular substitution, so
// the latency-bound parts of the two stages overlap.  Per chunk:
//   A: X = ... K S^T (waves 0,1) and O = diag(gamma) Q S^T (waves 2..5)   [chunk c]
//   S: stage chunk c+1 (fp16 tiles, transposed keys, gate tables); prefetch chunk c+2
//   B: U_i = T_ii (X_i - sum_{j<i} A_ij U_j) (waves 0,1)                   [chunk c]
//      A, P, T_ii of chunk c+1 (waves 2..7)
//   C: O += P U, write o (waves 2..5); S <- gamma S + U^T diag(.) K (all)  [chunk c]
// The products run on v_mfma_f32_16x16x32_f16 / 16x16x16_f16 with fp32 accumulation.
// bf16 inputs convert exactly to fp16 (|x| <= 65504); derived operands (S, P, U, T) are
// rounded to fp16, whose 11-bit significand keeps the bf16-output error budget.
// Decay factors: inside a 16-token diagonal block e^{G_r - G_j} is formed directly; across
// blocks it is split at the end of the previous block, e^{G_r - G_ref} * e^{G_ref - G_j},
// both factors <= 1, so no gate strength can overflow it.
#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>

#include "gdn_internal.h"
#include "gdn_mfma_common.h"

namespace gdn {
namespace {

using namespace mfma;

constexpr int D = 128;       // head dimension (d_k = d_v)
constexpr int C = 64;        // chunk length
constexpr int DVT = 32;      // value rows per workgroup
constexpr int NT = D / DVT;  // workgroups per stream
constexpr int NTH = 512;     // threads per workgroup (8 wavefronts)
constexpr int LQ = D + 8;    // row stride (halves) of [token][channel] tiles
constexpr int LC = C + 8;    // row stride (halves) of [channel][token] and [token][token] tiles
constexpr int LT = 24;       // row stride (halves) of 16x16 blocks

// Per-chunk gate tables (double-buffered with the chunk's other state-independent data).
struct alignas(16) Gates {
  alignas(16) float G[C];     // inclusive prefix of log alpha
  alignas(16) float gam[C];   // e^{G_r}
  alignas(16) float dec[C];   // e^{G_63 - G_r}
  alignas(16) float beta[C];
  alignas(16) float el[C];    // e^{G_r - G_ref(block of r)}, G_ref(R) = G_{16R-1} (0 for R = 0)
  alignas(16) float er[4][C]; // er[R][j] = e^{G_ref(R) - G_j} for j < 16 R
};

struct alignas(16) Smem {
  alignas(16) _Float16 q[C][LQ];           // queries of the staged chunk        [token][d_k]
  alignas(16) _Float16 k[C][LQ];           // keys of the staged chunk           [token][d_k]
  alignas(16) _Float16 kt[2][D][LC];       // keys transposed (swizzled)         [d_k][token]
  alignas(16) _Float16 s[DVT][LQ];         // fp16 copy of the state slice       [d_v][d_k]
  alignas(16) _Float16 p[2][C][LC];        // tril(Q K^T * D), inclusive          [token][token]
  alignas(16) _Float16 an[2][C][LC];       // -A, off-diagonal 16x16 blocks       [token][token]
  alignas(16) _Float16 td[2][4][16][LT];   // inverses of the diagonal blocks of (I + A), row-major
  alignas(16) _Float16 nt[4][16][LT];      // scratch: transposed diagonal blocks of A
  alignas(16) _Float16 u[DVT][LC];         // U                                   [d_v][token]
  alignas(16) _Float16 ud[DVT][LC];        // diag(e^{G_63 - G}) U                [d_v][token]
  alignas(16) _Float16 v[C][DVT + 8];      // value slice of the staged chunk     [token][d_v]
  alignas(16) Gates gt[2];
};

// ------------------------------------------------------------------------------------------
// Staging.  Global -> registers through buffer loads on per-stream buffer descriptors: the
// hardware range check returns zeros for tokens at or past the end of the stream, which pads
// a ragged last chunk with identity steps (k = v = q = 0, beta = 0, log alpha = 0) without
// branches, and buffer loads never touch the LDS counter, so waits on LDS traffic never wait
// for the prefetch.  Threads 0..255 stage keys (and values, gates), threads 256..511 queries.

struct Streams {
  __amdgpu_buffer_rsrc_t qk, v, beta, g;
};

__device__ __forceinline__ Streams make_streams(const ChunkArgs& p, int64_t bh, bool is_q) {
  const int64_t tok = bh * p.T;
  const int bytes_qkv = (int)(p.T * D * 2);
  const int bytes_tok = (int)(p.T * 2);
  const void* qk = is_q ? p.q : p.k;
  Streams s;
  s.qk = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)qk + tok * D), 0, bytes_qkv, kRsrcWord3);
  s.v = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)p.v + tok * D), 0, bytes_qkv, kRsrcWord3);
  s.beta = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)p.beta + tok), 0, bytes_tok, kRsrcWord3);
  s.g = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)p.log_alpha + tok), 0, bytes_tok, kRsrcWord3);
  return s;
}

struct Stage {
  v4u x[4];                // rows 4*(t/16)+i, channels 8*(t%16)..+7 (t = tid mod 256)
  v4u v;                   // key threads: row t/4, value channels c0 + 8*(t%4)..+7
  unsigned short beta, g;  // wavefront 0: token tid
};

__device__ __forceinline__ void stage_load(Stage& st, const Streams& sr, int64_t t0, int tid, int c0) {
  const int t = tid & 255;
  const int g8 = t & 15, rq = t >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    st.x[i] = __builtin_amdgcn_raw_buffer_load_b128(sr.qk, (int)(((t0 + 4 * rq + i) * D + 8 * g8) * 2), 0, 0);
  if (tid < 256)
    st.v = __builtin_amdgcn_raw_buffer_load_b128(sr.v, (int)(((t0 + (t >> 2)) * D + c0 + 8 * (t & 3)) * 2), 0, 0);
  if (tid < C) {
    st.beta = __builtin_amdgcn_raw_buffer_load_b16(sr.beta, (int)((t0 + tid) * 2), 0, 0);
    st.g = __builtin_amdgcn_raw_buffer_load_b16(sr.g, (int)((t0 + tid) * 2), 0, 0);
  }
}

// Register -> LDS: fp16 tiles (row-major keys and queries, transposed keys into buffer b)
// and the gate tables of buffer b.
__device__ __forceinline__ void stage_store(const Stage& st, Smem& sm, int b, int tid) {
  const int t = tid & 255;
  const int g8 = t & 15, rq = t >> 4;
  if (tid >= 256) {
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<h8*>(&sm.q[4 * rq + i][8 * g8]) = bf8_to_h8(st.x[i]);
    return;
  }
  h8 kh[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    kh[i] = bf8_to_h8(st.x[i]);
    *reinterpret_cast<h8*>(&sm.k[4 * rq + i][8 * g8]) = kh[i];
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    h4 col;
    col[0] = kh[0][e]; col[1] = kh[1][e]; col[2] = kh[2][e]; col[3] = kh[3][e];
    *reinterpret_cast<h4*>(&sm.kt[b][8 * g8 + e][kt_col(8 * g8 + e, 4 * rq)]) = col;
  }
  *reinterpret_cast<h8*>(&sm.v[t >> 2][8 * (t & 3)]) = bf8_to_h8(st.v);
  if (tid < C) {
    const float x = wave_prefix_sum(__uint_as_float(static_cast<uint32_t>(st.g) << 16));
    const float glast = __shfl(x, C - 1, 64);
    const float gr1 = __shfl(x, 15, 64), gr2 = __shfl(x, 31, 64), gr3 = __shfl(x, 47, 64);
    const int R = tid >> 4;
    const float gref = R == 0 ? 0.f : (R == 1 ? gr1 : (R == 2 ? gr2 : gr3));
    Gates& g = sm.gt[b];
    g.G[tid] = x;
    g.gam[tid] = __expf(x);
    g.dec[tid] = __expf(glast - x);
    g.beta[tid] = __uint_as_float(static_cast<uint32_t>(st.beta) << 16);
    g.el[tid] = __expf(x - gref);
    g.er[1][tid] = __expf(fminf(gr1 - x, 0.f));
    g.er[2][tid] = __expf(fminf(gr2 - x, 0.f));
    g.er[3][tid] = __expf(fminf(gr3 - x, 0.f));
  }
}

// ------------------------------------------------------------------------------------------
// State-independent products of one chunk (buffer b).  A Gram job is a 16x16 tile (R, J) of A
// (kind 0, from K K^T) or of P (kind 1, from Q K^T), computed as (M = j, N = r) so the lane
// holds a row of the tile: r = 16 R + lr, j = 16 J + 4 lg + i.
template <int KIND>
__device__ __forceinline__ f4 gram_scale(const Gates& g, int R, int J, int lr, int lg, f4 acc) {
  const int r = 16 * R + lr, j0 = 16 * J + 4 * lg;
  f4 f;
  if (R == J) {
    const float gr = g.G[r];
    const f4 gj = *reinterpret_cast<const f4*>(&g.G[j0]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = j0 + i;
      const bool keep = KIND ? (j <= r) : (j < r);
      const float e = __expf(fminf(gr - gj[i], 0.f));  // <= 1; masked entries are dropped below
      f[i] = keep ? e : 0.f;
    }
  } else {
    f = g.el[r] * *reinterpret_cast<const f4*>(&g.er[R][j0]);
  }
  return KIND == 0 ? (g.beta[r] * f) * acc : f * acc;
}

// Inverse of the unit lower-triangular diagonal block (I + N), N = A_JJ strictly lower, as
// (I - N)(I + N^2)(I + N^4)(I + N^8) (N^16 = 0) on 16x16x16 MFMAs.  With row(M) (lane holds
// M[lr][4lg..+3], the A-operand layout) and col(M) (lane holds M[4lg..+3][lr], the B-operand
// and accumulator layout): col(XY) = mfma(row X, col Y) and row(XY) = mfma(col Y, row X).
// rowN arrives in registers; colN goes through an LDS transpose private to this wavefront.
__device__ __forceinline__ void invert_diag(Smem& sm, int b, int J, f4 rowN, int lr, int lg) {
  const f4 zero = {0.f, 0.f, 0.f, 0.f};
  f4 eye;  // identity in either layout: element i of lane (lr, lg) is on the diagonal iff 4 lg + i == lr
#pragma unroll
  for (int i = 0; i < 4; ++i) eye[i] = (4 * lg + i == lr) ? 1.f : 0.f;
  const h4 rN = to_h4(rowN);
#pragma unroll
  for (int i = 0; i < 4; ++i) sm.nt[J][4 * lg + i][lr] = rN[i];
  // the transpose is written and read by this wavefront only: order the LDS accesses
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const h4 cN = *reinterpret_cast<const h4*>(&sm.nt[J][lr][4 * lg]);
  const f4 n2c = mfma16(rN, cN, zero), n2r = mfma16(cN, rN, zero);
  const h4 n2ch = to_h4(n2c), n2rh = to_h4(n2r);
  const f4 n4c = mfma16(n2rh, n2ch, zero), n4r = mfma16(n2ch, n2rh, zero);
  const f4 n8c = mfma16(to_h4(n4r), to_h4(n4c), zero);
  const f4 p1r = mfma16(to_h4(n2c + eye), to_h4(eye - rowN), zero);
  const f4 p2r = mfma16(to_h4(n4c + eye), to_h4(p1r), zero);
  const f4 tr = mfma16(to_h4(n8c + eye), to_h4(p2r), zero);
  *reinterpret_cast<h4*>(&sm.td[b][J][lr][4 * lg]) = to_h4(tr);
}

// Job codes: kind << 4 | R << 2 | J.  Each producing wavefront takes up to four jobs; jobs of
// one column J reuse the key fragment of block J, loaded once per 32-channel step.
constexpr int job(int kind, int R, int J) { return (kind << 4) | (R << 2) | J; }
constexpr int kNone = -1;

template <int J0, int J1, int J2, int J3>
__device__ __forceinline__ void gram_jobs(Smem& sm, int b, int l) {
  constexpr int jobs[4] = {J0, J1, J2, J3};
  const int lr = l & 15, lg = l >> 4;
  f4 acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (jobs[t] == kNone) continue;
      const int kind = jobs[t] >> 4, R = (jobs[t] >> 2) & 3, J = jobs[t] & 3;
      const _Float16* Bm = kind ? &sm.q[0][0] : &sm.k[0][0];
      acc[t] = mfma32(frag8(&sm.k[0][0], LQ, 16 * J, 32 * kk, l), frag8(Bm, LQ, 16 * R, 32 * kk, l), acc[t]);
    }
  }
  const Gates& g = sm.gt[b];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    if (jobs[t] == kNone) continue;
    const int kind = jobs[t] >> 4, R = (jobs[t] >> 2) & 3, J = jobs[t] & 3;
    const int r = 16 * R + lr, j0 = 16 * J + 4 * lg;
    if (kind == 1) {
      *reinterpret_cast<h4*>(&sm.p[b][r][j0]) = to_h4(gram_scale<1>(g, R, J, lr, lg, acc[t]));
    } else {
      const f4 a = gram_scale<0>(g, R, J, lr, lg, acc[t]);
      if (R == J)
        invert_diag(sm, b, J, a, lr, lg);
      else
        *reinterpret_cast<h4*>(&sm.an[b][r][j0]) = to_h4(-a);
    }
  }
}

// Producer wavefronts 2..7: the 20 tiles of A and P plus the four diagonal inverses.
__device__ __forceinline__ void produce(Smem& sm, int b, int w, int l) {
  switch (w) {
    case 2: gram_jobs<job(0, 0, 0), job(0, 1, 0), job(0, 2, 0), job(0, 3, 0)>(sm, b, l); break;
    case 3: gram_jobs<job(1, 0, 0), job(1, 1, 0), job(1, 2, 0), job(1, 3, 0)>(sm, b, l); break;
    case 4: gram_jobs<job(0, 1, 1), job(0, 2, 1), job(0, 3, 1), job(1, 1, 1)>(sm, b, l); break;
    case 5: gram_jobs<job(1, 2, 1), job(1, 3, 1), job(0, 2, 2), kNone>(sm, b, l); break;
    case 6: gram_jobs<job(1, 3, 2), job(0, 3, 3), kNone, kNone>(sm, b, l); break;
    default: gram_jobs<job(1, 2, 2), job(0, 3, 2), job(1, 3, 3), kNone>(sm, b, l); break;
  }
}

template <typename TOut>
__global__ __launch_bounds__(NTH, 1) void gdn_chunk_mfma_kernel(ChunkArgs p) {
  __shared__ Smem sm;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  int l = tid & 63;

  // XCD-aware placement: consecutive workgroup ids are dealt round-robin over the 8 XCDs;
  // remap so the NT slices of a stream get ids that land on the same XCD.
  const unsigned nblk = gridDim.x;
  unsigned bid = blockIdx.x;
  if (nblk % (8 * NT) == 0) bid = (bid % 8) * (nblk / 8) + bid / 8;
  const int tile = bid % NT;
  const int64_t bh = bid / NT;
  const int c0 = tile * DVT;
  const int64_t T = p.T;
  const int64_t nchunks = (T + C - 1) / C;

  // zero the never-written upper blocks of P and -A once
  for (int e = tid; e < 2 * C * LC; e += NTH) {
    (&sm.p[0][0][0])[e] = (_Float16)0.f;
    (&sm.an[0][0][0])[e] = (_Float16)0.f;
  }

  // state slice: wavefront w holds the S^T tiles (d_k block w, d_v block db): lane holds
  // S[dv = 16 db + lr][dk = 16 w + 4 lg .. +3]
  f4 S[2];
  {
    const int lr = l & 15, lg = l >> 4;
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const int dk = 16 * w + 4 * lg, dv = 16 * db + lr;
      f4 x = {0.f, 0.f, 0.f, 0.f};
      if (p.s0) x = *reinterpret_cast<const f4*>(p.s0 + (bh * D + c0 + dv) * D + dk);
      S[db] = x;
      *reinterpret_cast<h4*>(&sm.s[dv][dk]) = to_h4(x);
    }
  }

  const Streams sr = make_streams(p, bh, tid >= 256);
  Stage st;
  if (nchunks > 0) {
    stage_load(st, sr, 0, tid, c0);
    __syncthreads();  // P / -A zeroed before the producers write into them
    stage_store(st, sm, 0, tid);
    if (nchunks > 1) stage_load(st, sr, C, tid, c0);
    __syncthreads();
    if (w >= 2) produce(sm, 0, w, l);
    __syncthreads();
  }

  TOut* O = static_cast<TOut*>(p.o);
  for (int64_t ci = 0; ci < nchunks; ++ci) {
    const int cb = (int)(ci & 1), nb = cb ^ 1;
    const int64_t t0 = ci * C;
    const int n = (int)(T - t0 < C ? T - t0 : C);
    const Gates& gc = sm.gt[cb];

    // ---- A: X tiles (waves 0,1: value block db = w) and O = diag(gamma) Q S^T (waves 2..5:
    // token block w - 2, both value blocks)
    l = opaque(l);
    int lr = l & 15, lg = l >> 4;
    f4 X[4], Oacc[2];
    if (w < 2) {
      const int db = w, dv = 16 * db + lr;
#pragma unroll
      for (int i = 0; i < 4; ++i) X[i] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const h8 sb = frag8(&sm.s[0][0], LQ, 16 * db, 32 * kk, l);
#pragma unroll
        for (int i = 0; i < 4; ++i) X[i] = mfma32(frag8(&sm.k[0][0], LQ, 16 * i, 32 * kk, l), sb, X[i]);
      }
      // lane: token c = 16 i + 4 lg + e, value channel dv
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = 16 * i + 4 * lg;
        const f4 be = *reinterpret_cast<const f4*>(&gc.beta[c]);
        const f4 ga = *reinterpret_cast<const f4*>(&gc.gam[c]);
#pragma unroll
        for (int e = 0; e < 4; ++e) X[i][e] = be[e] * ((float)sm.v[c + e][dv] - ga[e] * X[i][e]);
      }
    } else if (w < 6) {
      const int cbk = w - 2;
      Oacc[0] = Oacc[1] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const h8 qb = frag8(&sm.q[0][0], LQ, 16 * cbk, 32 * kk, l);
#pragma unroll
        for (int db = 0; db < 2; ++db) Oacc[db] = mfma32(frag8(&sm.s[0][0], LQ, 16 * db, 32 * kk, l), qb, Oacc[db]);
      }
      // lane: value channel dv = 16 db + 4 lg + e, token c = 16 cbk + lr
      const float ga = gc.gam[16 * cbk + lr];
      Oacc[0] *= ga;
      Oacc[1] *= ga;
    }
    __syncthreads();

    // ---- S: stage chunk ci+1 into the other buffer, prefetch chunk ci+2
    if (ci + 1 < nchunks) {
      stage_store(st, sm, nb, tid);
      if (ci + 2 < nchunks) stage_load(st, sr, t0 + 2 * C, tid, c0);
    }
    __syncthreads();

    // ---- B: substitution of chunk ci (waves 0,1); A, P, T_ii of chunk ci+1 (waves 2..7)
    l = opaque(l);
    lr = l & 15, lg = l >> 4;
    if (w < 2) {
      const int db = w, dv = 16 * db + lr;
      h4 an[6], tdf[4];
#pragma unroll
      for (int i = 0, m = 0; i < 4; ++i) {
        tdf[i] = frag4(&sm.td[cb][i][0][0], LT, 0, 0, l);
#pragma unroll
        for (int j = 0; j < i; ++j, ++m) an[m] = frag4(&sm.an[cb][0][0], LC, 16 * i, 16 * j, l);
      }
      h4 Uh[4];
#pragma unroll
      for (int i = 0, m = 0; i < 4; ++i) {
        f4 acc = X[i];
#pragma unroll
        for (int j = 0; j < i; ++j, ++m) acc = mfma16(an[m], Uh[j], acc);
        const f4 U = mfma16(tdf[i], to_h4(acc), f4{0.f, 0.f, 0.f, 0.f});
        Uh[i] = to_h4(U);
        // lane: token c = 16 i + 4 lg + e, value channel dv
        const int cbase = 16 * i + 4 * lg;
        *reinterpret_cast<h4*>(&sm.u[dv][cbase]) = Uh[i];
        *reinterpret_cast<h4*>(&sm.ud[dv][cbase]) = to_h4(U * *reinterpret_cast<const f4*>(&gc.dec[cbase]));
      }
    } else if (ci + 1 < nchunks) {
      produce(sm, nb, w, l);
    }
    __syncthreads();

    // ---- C: O += U^T P^T and the output (waves 2..5); the state hand-off (all)
    l = opaque(l);
    lr = l & 15, lg = l >> 4;
    if (w >= 2 && w < 6) {
      const int cbk = w - 2;
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        if (kc == 1 && cbk < 2) continue;
        const h8 pb = frag8(&sm.p[cb][0][0], LC, 16 * cbk, 32 * kc, l);
#pragma unroll
        for (int db = 0; db < 2; ++db) Oacc[db] = mfma32(frag8(&sm.u[0][0], LC, 16 * db, 32 * kc, l), pb, Oacc[db]);
      }
      const int c = 16 * cbk + lr;
      if (c < n) {
#pragma unroll
        for (int db = 0; db < 2; ++db) store_o4<TOut>(O, (bh * T + t0 + c) * D + c0 + 16 * db + 4 * lg, Oacc[db]);
      }
    }
    {
      const float glast = gc.gam[C - 1];
      const bool snap = p.s_ckpt && n == C && ((t0 + n) % p.ckpt_every) == 0;
      const int dkr = 16 * w + lr;  // key channel of this lane's A-operand row
      h8 ka[2];
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) ka[kc] = *reinterpret_cast<const h8*>(&sm.kt[cb][dkr][kt_col(dkr, 32 * kc + 8 * lg)]);
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        f4 acc = S[db] * glast;
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) acc = mfma32(ka[kc], frag8(&sm.ud[0][0], LC, 16 * db, 32 * kc, l), acc);
        S[db] = acc;
        const int dk = 16 * w + 4 * lg, dv = 16 * db + lr;
        *reinterpret_cast<h4*>(&sm.s[dv][dk]) = to_h4(acc);
        if (snap) {
          const int64_t idx = (t0 + n) / p.ckpt_every - 1;
          *reinterpret_cast<f4*>(p.s_ckpt + ((bh * p.n_ckpt + idx) * D + c0 + dv) * D + dk) = acc;
        }
      }
    }
    __syncthreads();
  }

  if (p.s_final) {
    const int lr = l & 15, lg = l >> 4;
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const int dk = 16 * w + 4 * lg, dv = 16 * db + lr;
      *reinterpret_cast<f4*>(p.s_final + (bh * D + c0 + dv) * D + dk) = S[db];
    }
  }
}

}  // namespace

bool chunk_mfma_supported(const ChunkArgs& a) {
  // buffer-descriptor offsets are 32-bit: one stream's q/k/v must stay under 2 GiB
  return a.in_dtype == GDN_BF16 && a.D == D && a.chunk == C && a.T * D * 2 < (INT64_C(1) << 31);
}

hipError_t launch_chunk_mfma(const ChunkArgs& a, bool kda, hipStream_t s) {
  if (kda) return launch_kda_mfma(a, s);
  const int64_t blocks = a.B * a.H * NT;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (a.out_dtype == GDN_BF16)
    hipLaunchKernelGGL((gdn_chunk_mfma_kernel<__hip_bfloat16>), dim3((unsigned)blocks), dim3(NTH), 0, s, a);
  else
    hipLaunchKernelGGL((gdn_chunk_mfma_kernel<float>), dim3((unsigned)blocks), dim3(NTH), 0, s, a);
  return hipGetLastError();
}

}  // namespace gdn
