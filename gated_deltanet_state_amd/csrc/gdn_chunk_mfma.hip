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
// Work decomposition (one workgroup = 4 wavefronts of 64 lanes):
//  * a workgroup owns one (batch, head) stream and a 32-row slice of the value channels
//    (the recurrence multiplies S only from the right, so value rows evolve independently);
//    the four slices of a stream are placed on the same XCD so they share its L2.
//  * the state slice lives in MFMA accumulators (fp32) for the whole sequence; a
//    half-precision copy in LDS is the operand of the state-coupled products.
//  * all products run on v_mfma_f32_16x16x32_f16 with fp32 accumulation.  bf16 inputs
//    convert exactly to fp16 (|x| <= 65504); derived operands (S, P, U) are rounded to
//    fp16, whose 11-bit significand keeps the bf16-output error budget.
//  * the triangular system is solved without forming (I + A)^-1: the four 16x16 diagonal
//    blocks are inverted by fp32 forward substitution, then U is built block row by block
//    row, U_i = T_ii (X_i - sum_{j<i} A_ij U_j), on v_mfma_f32_16x16x16_f16 -- whose
//    accumulator lane layout equals its B-operand layout, so each U_j feeds the next
//    product from registers.
//  * decay factors: within a 16-token diagonal block e^{G_r - G_j} is formed directly;
//    across blocks it is split at the end of the previous block, e^{G_r - G_ref} *
//    e^{G_ref - G_j}, both factors <= 1, so no gate strength can overflow it.
//  * the next chunk's inputs are loaded into registers while the current chunk computes.
#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>

#include "gdn_internal.h"

namespace gdn {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

constexpr int D = 128;       // head dimension (d_k = d_v)
constexpr int C = 64;        // chunk length
constexpr int DVT = 32;      // value rows per workgroup
constexpr int NT = D / DVT;  // workgroups per stream
constexpr int NTH = 256;     // threads per workgroup
constexpr int LQ = D + 8;    // row stride (halves) of [token][channel] tiles
constexpr int LC = C + 8;    // row stride (halves) of [channel][token] tiles
constexpr int LT = 24;       // row stride (halves) of the 16x16 diagonal inverse blocks
constexpr int LA = 20;       // row stride (floats) of the 16x16 fp32 diagonal A blocks

struct Smem {
  _Float16 q[C][LQ];        // queries of the chunk            [token][d_k]
  _Float16 k[C][LQ];        // keys                            [token][d_k]
  _Float16 kt[D][LC];       // keys transposed                 [d_k][token]
  _Float16 s[DVT][LQ];      // fp16 copy of the state slice    [d_v][d_k]
  _Float16 p[C][LC];        // tril(Q K^T * D), inclusive       [token][token]
  _Float16 an[C][LC];       // -A, off-diagonal 16x16 blocks    [token][token]
  _Float16 u[DVT][LC];      // U                               [d_v][token]
  _Float16 ud[DVT][LC];     // diag(e^{G_63 - G}) U            [d_v][token]
  _Float16 v[C][DVT + 8];   // value slice                     [token][d_v]
  _Float16 td[4][16][LT];   // inverses of the diagonal blocks of (I + A)
  float ad[4][16][LA];      // diagonal blocks of A (fp32)
  float G[C];               // inclusive prefix of log alpha
  float gam[C];             // e^{G_r}
  float dec[C];             // e^{G_63 - G_r}
  float beta[C];
  float el[C];              // e^{G_r - G_ref(block of r)}
  float er[4][C];           // er[R][j] = e^{G_ref(R) - G_j}, j < 16 R
};

__device__ __forceinline__ f4 mfma32(h8 a, h8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 mfma16(h4 a, h4 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

// Returns x unchanged but opaque to the optimiser, so per-lane addresses derived from it are
// recomputed where they are used instead of being hoisted out of the chunk loop and kept
// live across every phase (which would exhaust the 256 architectural registers).
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Operand fragment of a 16 x 32 slice (rows m0.., columns k0..) of a row-major fp16 matrix:
// lane l holds row m0 + l%16, columns k0 + 8*(l/16) .. +7.  Used for both MFMA operands
// (for B the "rows" are the N index).
__device__ __forceinline__ h8 frag8(const _Float16* base, int ld, int m0, int k0, int lane) {
  return *reinterpret_cast<const h8*>(base + (m0 + (lane & 15)) * ld + k0 + 8 * (lane >> 4));
}
// Same for a 16 x 16 slice and the 16x16x16 instruction: columns k0 + 4*(l/16) .. +3.
__device__ __forceinline__ h4 frag4(const _Float16* base, int ld, int m0, int k0, int lane) {
  return *reinterpret_cast<const h4*>(base + (m0 + (lane & 15)) * ld + k0 + 4 * (lane >> 4));
}

// The transposed-key tile kt[d_k][token] stores its 16-byte groups of 8 tokens XOR-swizzled
// by bits 3..5 of the key channel, so that the staging writes (16 lanes writing 16 channels
// 8 apart, same tokens) spread over the LDS banks; 16-byte reads stay contiguous.
__device__ __forceinline__ int kt_col(int dk, int c) { return (((c >> 3) ^ ((dk >> 3) & 7)) << 3) | (c & 7); }

__device__ __forceinline__ h4 to_h4(f4 x) {
  h4 r;
  r[0] = (_Float16)x[0]; r[1] = (_Float16)x[1]; r[2] = (_Float16)x[2]; r[3] = (_Float16)x[3];
  return r;
}

// 8 bf16 (packed in 4 dwords, element 2i in the low half) -> 8 fp16 (exact for |x| <= 65504)
__device__ __forceinline__ h8 bf8_to_h8(v4u x) {
  const uint32_t w[4] = {x[0], x[1], x[2], x[3]};
  h8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[2 * i] = (_Float16)__uint_as_float(w[i] << 16);
    r[2 * i + 1] = (_Float16)__uint_as_float(w[i] & 0xffff0000u);
  }
  return r;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const uint32_t lo = __bfloat16_as_ushort(__float2bfloat16(a));
  const uint32_t hi = __bfloat16_as_ushort(__float2bfloat16(b));
  return lo | (hi << 16);
}

// Global -> register staging of one chunk's inputs, through buffer loads on per-stream
// buffer descriptors: the hardware range check returns zeros for tokens at or past the end
// of the stream, which pads a ragged last chunk with identity steps (k = v = q = 0,
// beta = 0, log alpha = 0) without branches, and buffer loads never touch the LDS
// counter, so waits on LDS traffic never wait for the prefetch.
constexpr int kRsrcWord3 = 0x00020000;  // gfx9-family raw buffer: 32-bit dwords, no swizzle

struct Streams {
  __amdgpu_buffer_rsrc_t q, k, v, beta, g;
};

__device__ __forceinline__ Streams make_streams(const ChunkArgs& p, int64_t bh) {
  const int64_t tok = bh * p.T;
  const int bytes_qkv = (int)(p.T * D * 2);
  const int bytes_tok = (int)(p.T * 2);
  Streams s;
  s.q = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)p.q + tok * D), 0, bytes_qkv, kRsrcWord3);
  s.k = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)p.k + tok * D), 0, bytes_qkv, kRsrcWord3);
  s.v = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)p.v + tok * D), 0, bytes_qkv, kRsrcWord3);
  s.beta = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)p.beta + tok), 0, bytes_tok, kRsrcWord3);
  s.g = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)p.log_alpha + tok), 0, bytes_tok, kRsrcWord3);
  return s;
}

struct Stage {
  v4u q[4], k[4];      // rows 4*(tid/16)+i, channels 8*(tid%16)..+7 (bf16 pairs)
  v4u v;               // row tid/4, value channels c0 + 8*(tid%4)..+7
  unsigned short beta, g;  // token tid (threads 0..63)
};

__device__ __forceinline__ void stage_load(Stage& st, const Streams& sr, int64_t t0, int tid, int c0) {
  const int g8 = tid & 15, rq = tid >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int off = (int)(((t0 + 4 * rq + i) * D + 8 * g8) * 2);
    st.q[i] = __builtin_amdgcn_raw_buffer_load_b128(sr.q, off, 0, 0);
    st.k[i] = __builtin_amdgcn_raw_buffer_load_b128(sr.k, off, 0, 0);
  }
  st.v = __builtin_amdgcn_raw_buffer_load_b128(sr.v, (int)(((t0 + (tid >> 2)) * D + c0 + 8 * (tid & 3)) * 2), 0, 0);
  if (tid < C) {
    st.beta = __builtin_amdgcn_raw_buffer_load_b16(sr.beta, (int)((t0 + tid) * 2), 0, 0);
    st.g = __builtin_amdgcn_raw_buffer_load_b16(sr.g, (int)((t0 + tid) * 2), 0, 0);
  }
}

// Register -> LDS: fp16 tiles (row-major and transposed keys) and the per-token gate tables.
__device__ __forceinline__ void stage_store(const Stage& st, Smem& sm, int tid) {
  const int g8 = tid & 15, rq = tid >> 4;
  h8 kh[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 4 * rq + i;
    *reinterpret_cast<h8*>(&sm.q[row][8 * g8]) = bf8_to_h8(st.q[i]);
    kh[i] = bf8_to_h8(st.k[i]);
    *reinterpret_cast<h8*>(&sm.k[row][8 * g8]) = kh[i];
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    h4 col;
    col[0] = kh[0][e]; col[1] = kh[1][e]; col[2] = kh[2][e]; col[3] = kh[3][e];
    *reinterpret_cast<h4*>(&sm.kt[8 * g8 + e][kt_col(8 * g8 + e, 4 * rq)]) = col;
  }
  *reinterpret_cast<h8*>(&sm.v[tid >> 2][8 * (tid & 3)]) = bf8_to_h8(st.v);
  if (tid < C) {
    // wavefront 0: inclusive prefix sum of log alpha over the 64 tokens
    float x = __uint_as_float(static_cast<uint32_t>(st.g) << 16);
#pragma unroll
    for (int off = 1; off < C; off <<= 1) {
      const float y = __shfl_up(x, off, 64);
      if (tid >= off) x += y;
    }
    const float glast = __shfl(x, C - 1, 64);
    const float gr1 = __shfl(x, 15, 64), gr2 = __shfl(x, 31, 64), gr3 = __shfl(x, 47, 64);
    const int R = tid >> 4;
    const float gref = R == 0 ? 0.f : (R == 1 ? gr1 : (R == 2 ? gr2 : gr3));
    sm.G[tid] = x;
    sm.gam[tid] = __expf(x);
    sm.dec[tid] = __expf(glast - x);
    sm.beta[tid] = __uint_as_float(static_cast<uint32_t>(st.beta) << 16);
    sm.el[tid] = __expf(x - gref);
    sm.er[1][tid] = tid < 16 ? __expf(gr1 - x) : 0.f;
    sm.er[2][tid] = tid < 32 ? __expf(gr2 - x) : 0.f;
    sm.er[3][tid] = tid < 48 ? __expf(gr3 - x) : 0.f;
  }
}

// Epilogue of one Gram tile held as (M = j, N = r): lane holds j = 16 J + 4 lg + i, r = 16 R + lr.
// KIND 0: A block -> fp32 diagonal block or fp16 -A off the diagonal; KIND 1: P block (fp16).
template <int KIND>
__device__ __forceinline__ void gram_epilogue(Smem& sm, int R, int J, int lr, int lg, f4 acc) {
  const int r = 16 * R + lr, j0 = 16 * J + 4 * lg;
  f4 f;
  if (R == J) {
    const float gr = sm.G[r];
    const f4 gj = *reinterpret_cast<const f4*>(&sm.G[j0]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = j0 + i;
      const bool keep = KIND ? (j <= r) : (j < r);
      const float e = __expf(fminf(gr - gj[i], 0.f));  // <= 1; masked entries are dropped below
      f[i] = keep ? e : 0.f;
    }
  } else {
    f = sm.el[r] * *reinterpret_cast<const f4*>(&sm.er[R][j0]);
  }
  if (KIND == 0) {
    const f4 a = (sm.beta[r] * f) * acc;
    if (R == J)
      *reinterpret_cast<f4*>(&sm.ad[R][lr][4 * lg]) = a;
    else
      *reinterpret_cast<h4*>(&sm.an[r][j0]) = to_h4(-a);
  } else {
    *reinterpret_cast<h4*>(&sm.p[r][j0]) = to_h4(f * acc);
  }
}

// Column block J of A and P: tiles (R, J), R = J..3.  The key fragment of block J is loaded
// once per 32-channel step and reused by all 2 (4 - J) tiles of the column.
template <int J>
__device__ __forceinline__ void gram_column(Smem& sm, int l, int lr, int lg) {
  constexpr int NR = 4 - J;
  f4 accA[NR], accP[NR];
#pragma unroll
  for (int t = 0; t < NR; ++t) {
    accA[t] = f4{0.f, 0.f, 0.f, 0.f};
    accP[t] = f4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const h8 a = frag8(&sm.k[0][0], LQ, 16 * J, 32 * kk, l);
#pragma unroll
    for (int t = 0; t < NR; ++t) {
      accA[t] = mfma32(a, frag8(&sm.k[0][0], LQ, 16 * (J + t), 32 * kk, l), accA[t]);
      accP[t] = mfma32(a, frag8(&sm.q[0][0], LQ, 16 * (J + t), 32 * kk, l), accP[t]);
    }
  }
#pragma unroll
  for (int t = 0; t < NR; ++t) {
    gram_epilogue<0>(sm, J + t, J, lr, lg, accA[t]);
    gram_epilogue<1>(sm, J + t, J, lr, lg, accP[t]);
  }
}

// Inverse of the unit lower-triangular diagonal block (I + A_JJ) by fp32 forward
// substitution, T[r][n] = delta_rn - sum_{j<r} A[r][j] T[j][n]; lane n < 16 owns column n
// (entries above the diagonal come out zero because T[j][n] = 0 for j < n).  Called by the
// wavefront that wrote A_JJ, so its own LDS writes are already ordered before these reads.
__device__ __forceinline__ void invert_diag(Smem& sm, int J, int l) {
  if (l < 16) {
    float t[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float arow[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f4 x = *reinterpret_cast<const f4*>(&sm.ad[J][r][4 * q]);
        arow[4 * q] = x[0]; arow[4 * q + 1] = x[1]; arow[4 * q + 2] = x[2]; arow[4 * q + 3] = x[3];
      }
      float acc = (r == l) ? 1.f : 0.f;
#pragma unroll
      for (int j = 0; j < r; ++j) acc -= arow[j] * t[j];
      t[r] = acc;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) sm.td[J][r][l] = (_Float16)t[r];
  }
}

// Output tiles O^T (token block cb, value block db) owned by wavefront w: w even owns one,
// w odd three, so that every wavefront issues the same number of products in phase 1.
__device__ __forceinline__ int o_tiles(int w) { return (w & 1) ? 3 : 1; }
__device__ __forceinline__ void o_tile(int w, int t, int& cb, int& db) {
  const int idx = (w & 1) ? t + 1 : 0;
  cb = 2 * (w >> 1) + (idx >> 1);
  db = idx & 1;
}

template <typename TOut>
__device__ __forceinline__ void store_o4(TOut* o, int64_t idx, f4 x);
template <>
__device__ __forceinline__ void store_o4<float>(float* o, int64_t idx, f4 x) {
  *reinterpret_cast<f4*>(o + idx) = x;
}
template <>
__device__ __forceinline__ void store_o4<__hip_bfloat16>(__hip_bfloat16* o, int64_t idx, f4 x) {
  uint2 w;
  w.x = pack_bf16x2(x[0], x[1]);
  w.y = pack_bf16x2(x[2], x[3]);
  *reinterpret_cast<uint2*>(o + idx) = w;
}

template <typename TOut>
__global__ __launch_bounds__(NTH, 1) void gdn_chunk_mfma_kernel(ChunkArgs p) {
  __shared__ Smem sm;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  int l = tid & 63;
  int lr = l & 15, lg = l >> 4;  // lane row / lane group in MFMA layouts

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
  for (int e = tid; e < C * LC; e += NTH) {
    (&sm.p[0][0])[e] = (_Float16)0.f;
    (&sm.an[0][0])[e] = (_Float16)0.f;
  }

  // state slice: wavefront w holds S^T tiles (d_k block kb = 2w + a, d_v block db): lane holds
  // S[dv = 16 db + lr][dk = 16 kb + 4 lg .. +3]
  f4 S[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const int dk = 16 * (2 * w + a) + 4 * lg, dv = 16 * db + lr;
      f4 x = {0.f, 0.f, 0.f, 0.f};
      if (p.s0) x = *reinterpret_cast<const f4*>(p.s0 + (bh * D + c0 + dv) * D + dk);
      S[a][db] = x;
      *reinterpret_cast<h4*>(&sm.s[dv][dk]) = to_h4(x);
    }

  const Streams sr = make_streams(p, bh);
  Stage st;
  if (nchunks > 0) {
    stage_load(st, sr, 0, tid, c0);
    stage_store(st, sm, tid);
  }
  __syncthreads();

  TOut* O = static_cast<TOut*>(p.o);
  for (int64_t ci = 0; ci < nchunks; ++ci) {
    const int64_t t0 = ci * C;
    const int n = (int)(T - t0 < C ? T - t0 : C);
    const bool more = ci + 1 < nchunks;
    if (more) stage_load(st, sr, t0 + C, tid, c0);

    // ---- phase 1: Gram column J = w, value tiles X (waves 2, 3), O = diag(gamma) Q S^T tiles,
    // then the inverse of the diagonal block (I + A_ww)
    l = opaque(l), lr = l & 15, lg = l >> 4;
    switch (w) {
      case 0: gram_column<0>(sm, l, lr, lg); break;
      case 1: gram_column<1>(sm, l, lr, lg); break;
      case 2: gram_column<2>(sm, l, lr, lg); break;
      default: gram_column<3>(sm, l, lr, lg); break;
    }
    f4 X[4];
    if (w >= 2) {
      const int db = w - 2;
      const int dv = 16 * db + lr;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          acc = mfma32(frag8(&sm.k[0][0], LQ, 16 * i, 32 * kk, l), frag8(&sm.s[0][0], LQ, 16 * db, 32 * kk, l), acc);
        // lane: token c = 16 i + 4 lg + e, value channel dv
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int c = 16 * i + 4 * lg + e;
          X[i][e] = sm.beta[c] * ((float)sm.v[c][dv] - sm.gam[c] * acc[e]);
        }
      }
    }
    f4 Oacc[3];
    const int nO = o_tiles(w);
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      if (t < nO) {
        int cb, db;
        o_tile(w, t, cb, db);
        f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          acc = mfma32(frag8(&sm.s[0][0], LQ, 16 * db, 32 * kk, l), frag8(&sm.q[0][0], LQ, 16 * cb, 32 * kk, l), acc);
        // lane: value channel dv = 16 db + 4 lg + e, token c = 16 cb + lr
        Oacc[t] = acc * sm.gam[16 * cb + lr];
      }
    }
    invert_diag(sm, w, l);
    __syncthreads();

    // ---- phase 3: block forward substitution U_i = T_ii (X_i - sum_{j<i} A_ij U_j), waves 2, 3
    l = opaque(l), lr = l & 15, lg = l >> 4;
    if (w >= 2) {
      const int db = w - 2;
      const int dv = 16 * db + lr;
      h4 Uh[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f4 acc = X[i];
#pragma unroll
        for (int j = 0; j < i; ++j) acc = mfma16(frag4(&sm.an[0][0], LC, 16 * i, 16 * j, l), Uh[j], acc);
        const f4 zero = {0.f, 0.f, 0.f, 0.f};
        const f4 U = mfma16(frag4(&sm.td[i][0][0], LT, 0, 0, l), to_h4(acc), zero);
        Uh[i] = to_h4(U);
        // lane: token c = 16 i + 4 lg + e, value channel dv
        const int cbase = 16 * i + 4 * lg;
        *reinterpret_cast<h4*>(&sm.u[dv][cbase]) = Uh[i];
        f4 Ud;
#pragma unroll
        for (int e = 0; e < 4; ++e) Ud[e] = U[e] * sm.dec[cbase + e];
        *reinterpret_cast<h4*>(&sm.ud[dv][cbase]) = to_h4(Ud);
      }
    }
    __syncthreads();

    // ---- phase 4: O += U^T P^T on the owned output tiles, then the state hand-off
    l = opaque(l), lr = l & 15, lg = l >> 4;
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      if (t < nO) {
        int cb, db;
        o_tile(w, t, cb, db);
        f4 acc = Oacc[t];
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
          if (kc == 0 || cb >= 2)
            acc = mfma32(frag8(&sm.u[0][0], LC, 16 * db, 32 * kc, l), frag8(&sm.p[0][0], LC, 16 * cb, 32 * kc, l), acc);
        const int c = 16 * cb + lr;
        if (c < n) store_o4<TOut>(O, (bh * T + t0 + c) * D + c0 + 16 * db + 4 * lg, acc);
      }
    }
    const float glast = sm.gam[C - 1];
    const bool snap = p.s_ckpt && n == C && ((t0 + n) % p.ckpt_every) == 0;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const int kb = 2 * w + a;
        const int dkr = 16 * kb + lr;  // key channel of this lane's A-operand row
        f4 acc = S[a][db] * glast;
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
          const h8 ka = *reinterpret_cast<const h8*>(&sm.kt[dkr][kt_col(dkr, 32 * kc + 8 * lg)]);
          acc = mfma32(ka, frag8(&sm.ud[0][0], LC, 16 * db, 32 * kc, l), acc);
        }
        S[a][db] = acc;
        const int dk = 16 * kb + 4 * lg, dv = 16 * db + lr;
        *reinterpret_cast<h4*>(&sm.s[dv][dk]) = to_h4(acc);
        if (snap) {
          const int64_t idx = (t0 + n) / p.ckpt_every - 1;
          *reinterpret_cast<f4*>(p.s_ckpt + ((bh * p.n_ckpt + idx) * D + c0 + dv) * D + dk) = acc;
        }
      }
    __syncthreads();
    if (more) {
      stage_store(st, sm, tid);
      __syncthreads();
    }
  }

  if (p.s_final) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const int dk = 16 * (2 * w + a) + 4 * lg, dv = 16 * db + lr;
        *reinterpret_cast<f4*>(p.s_final + (bh * D + c0 + dv) * D + dk) = S[a][db];
      }
  }
}

}  // namespace

bool chunk_mfma_supported(const ChunkArgs& a) {
  // buffer-descriptor offsets are 32-bit: one stream's q/k/v must stay under 2 GiB
  return a.in_dtype == GDN_BF16 && a.D == D && a.chunk == C && a.T * D * 2 < (INT64_C(1) << 31);
}

hipError_t launch_chunk_mfma(const ChunkArgs& a, bool kda, hipStream_t s) {
  if (kda) return launch_chunk_valu(a, true, s);  // per-channel decay: vector path for now
  const int64_t blocks = a.B * a.H * NT;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (a.out_dtype == GDN_BF16)
    hipLaunchKernelGGL((gdn_chunk_mfma_kernel<__hip_bfloat16>), dim3((unsigned)blocks), dim3(NTH), 0, s, a);
  else
    hipLaunchKernelGGL((gdn_chunk_mfma_kernel<float>), dim3((unsigned)blocks), dim3(NTH), 0, s, a);
  return hipGetLastError();
}

}  // namespace gdn
