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
//   T = (I + A)^{-1}                                   unit lower triangular
//   X = diag(beta) (V - diag(gamma) K S^T)             (64 x d_v)
//   U = T X
//   O = diag(gamma) Q S^T + tril(Q K^T * D) U          outputs
//   S <- gamma_63 S + U^T diag(e^{G_63 - G}) K         state handed to the next chunk
//
// Work decomposition: a workgroup owns one (batch, head) stream and a 32-row slice of the
// value channels (the recurrence multiplies S only from the right, so value rows evolve
// independently); the four slices of a stream are placed on the same XCD so they share its
// L2.  Eight wavefronts take fixed roles (waves w and w + 4 share a SIMD):
//   0, 1  state chain: each keeps a 16 x 128 block of S in fp32 MFMA accumulators for the
//         whole sequence and runs X, U = T X and the state update with every operand
//         regrouped in registers (no LDS round trip on the chunk-to-chunk dependency);
//   4, 5  outputs of two 16-token blocks each: O = diag(gamma) Q S^T + P U;
//   6, 7  one chunk ahead: the diagonal 16x16 blocks of A, their inverses and the
//         off-diagonal blocks of T (wave 6); the off-diagonal blocks of A (wave 7); the
//         causal scores P = tril(Q K^T * D) (both);
//   2, 3  staging: keys (row-major, and transposed for the state update), queries, values
//         and the gate tables, converted to fp16 and written to LDS one or two chunks ahead.
// Each iteration has two barrier-separated phases; iteration c works on chunk c (chain,
// outputs), chunk c + 1 (producers) and chunks c + 1, c + 2 (staging).
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
constexpr int LQ = D + 16;   // row stride (halves) of [token][channel] tiles: 288 bytes = 72 banks
constexpr int LC = C + 8;    // row stride (halves) of [channel][token] and [token][token] tiles
constexpr int LT = 24;       // row stride (halves) of 16x16 blocks

// Per-chunk gate tables.
struct alignas(16) Gates {
  alignas(16) float G[C];     // inclusive prefix of log alpha
  alignas(16) float gam[C];   // e^{G_r}
  alignas(16) float dec[C];   // e^{G_63 - G_r}
  alignas(16) float beta[C];
  alignas(16) float el[C];    // e^{G_r - G_ref(block of r)}, G_ref(R) = G_{16R-1} (0 for R = 0)
  alignas(16) float nbel[C];  // -beta_r el_r
  alignas(16) float er[3][C]; // er[R-1][j] = e^{G_ref(R) - G_j} for j < 16 R, R = 1..3
};

// Buffers hold data of one chunk: keys and gate tables by chunk mod 3, the others by chunk
// mod 2.  Bank
// layout (gfx950 LDS: 16-byte accesses are served 32 lanes at a time over 128 four-byte banks):
// a 16-row x 32-column fragment read is conflict-free when the row stride is an odd multiple
// of 8 banks, hence the 288-byte rows of the [token][channel] tiles.
struct alignas(16) Smem {
  alignas(16) _Float16 k[3][C][LQ];      // keys                                  [token][d_k]
  alignas(16) _Float16 q[2][C][LQ];      // queries                               [token][d_k]
  alignas(16) _Float16 s[DVT][LQ];       // fp16 state slice entering the chain's chunk [d_v][d_k]
  alignas(16) uint16_t vt[2][DVT][LC];   // value slice, bf16 bits                [d_v][token]
  alignas(16) _Float16 t[2][C][LC];      // T = (I + A)^{-1}, upper blocks zero; A_JJ staged on the diagonal
  alignas(16) _Float16 p[2][C][LC];      // tril(Q K^T * D), upper blocks zero     [token][token]
  alignas(16) _Float16 an[6][16][LT];    // -A, off-diagonal blocks (R, J), R > J
  alignas(16) _Float16 u[DVT][LC];       // U of the chain's chunk                [d_v][token]
  alignas(16) Gates gt[3];
};
static_assert(sizeof(Smem) <= 160 * 1024, "LDS budget");
__device__ __forceinline__ int kbuf(int64_t chunk) { return (int)(((chunk % 3) + 3) % 3); }

constexpr int an_idx(int R, int J) { return R * (R - 1) / 2 + J; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t stream_rsrc(const void* base, int64_t elem0, int64_t n_elems) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)base + elem0), 0, (int)(n_elems * 2), kRsrcWord3);
}
__device__ __forceinline__ v4u ld_b128(__amdgpu_buffer_rsrc_t r, int64_t elem) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)(elem * 2), 0, 0);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ h8 lds8(const _Float16* p) { return *reinterpret_cast<const h8*>(p); }
__device__ __forceinline__ h4 lds4(const _Float16* p) { return *reinterpret_cast<const h4*>(p); }

// Dword m of the 16-bit transpose: halves e of dwords x (low result half) and y (high).
__device__ __forceinline__ uint32_t pick2(uint32_t x, uint32_t y, int e) {
  return __builtin_amdgcn_perm(y, x, (e & 1) ? 0x07060302u : 0x05040100u);
}

// ------------------------------------------------------------------------------------------
// Decay-weighted Gram tiles.  A tile (R, J) of A (from K K^T) or of P (from Q K^T) is computed
// as (M = j, N = r), so the lane holds a row of the tile: r = 16 R + lr, j = 16 J + 4 lg + e.
// Off the diagonal the decay splits at the reference point (both factors <= 1); on the
// diagonal the factor e^{G_r - G_j} (j <= r) is formed directly and shared by A and P.
__device__ __forceinline__ f4 offdiag_neg_a(const Gates& g, int R, int J, int lr, int lg, f4 acc) {
  const int r = 16 * R + lr;
  return (g.nbel[r] * *reinterpret_cast<const f4*>(&g.er[R - 1][16 * J + 4 * lg])) * acc;
}
__device__ __forceinline__ f4 offdiag_p(const Gates& g, int R, int J, int lr, int lg, f4 acc) {
  const int r = 16 * R + lr;
  return (g.el[r] * *reinterpret_cast<const f4*>(&g.er[R - 1][16 * J + 4 * lg])) * acc;
}
// e^{G_r - G_j} for r = 16 J + lr, j = 16 J + 4 lg + e, zero for j > r.
__device__ __forceinline__ f4 diag_decay(const Gates& g, int J, int lr, int lg) {
  const int r = 16 * J + lr, j0 = 16 * J + 4 * lg;
  const float gr = g.G[r];
  const f4 gj = *reinterpret_cast<const f4*>(&g.G[j0]);
  f4 f;
#pragma unroll
  for (int e = 0; e < 4; ++e) f[e] = (j0 + e <= r) ? __expf(gr - gj[e]) : 0.f;
  return f;
}

// Inverses of the four unit lower-triangular diagonal blocks (I + N_J), N_J = A_JJ strictly
// lower, as (I - N)(I + N^2)(I + N^4)(I + N^8) (N^16 = 0) on 16x16x16 MFMAs.  With row(M)
// (lane holds M[lr][4lg..+3], the A-operand layout) and col(M) (lane holds M[4lg..+3][lr], the
// B-operand and accumulator layout): col(XY) = mfma(row X, col Y) and row(XY) = mfma(col Y,
// row X); in particular col(N) = mfma(row N, col I).  Returns each inverse in both layouts
// (the factors commute, so either order is the product).  The four chains are independent
// and advance level by level so their MFMA latencies overlap.
__device__ __forceinline__ void invert_diag4(const f4 (&rowN)[4], int lr, int lg, h4 (&Tr)[4], h4 (&Tc)[4]) {
  const f4 zero = {0.f, 0.f, 0.f, 0.f};
  f4 eye;  // identity in either layout: element i of lane (lr, lg) is on the diagonal iff 4 lg + i == lr
#pragma unroll
  for (int i = 0; i < 4; ++i) eye[i] = (4 * lg + i == lr) ? 1.f : 0.f;
  const h4 eyeh = to_h4(eye);
  h4 rN[4], cN[4], n2ch[4], n2rh[4], n4ch[4], n4rh[4], p1[4], n8e[4], p2r[4];
  f4 n2c[4], n4c[4];
#pragma unroll
  for (int J = 0; J < 4; ++J) rN[J] = to_h4(rowN[J]);
#pragma unroll
  for (int J = 0; J < 4; ++J) cN[J] = to_h4(mfma16(rN[J], eyeh, zero));
#pragma unroll
  for (int J = 0; J < 4; ++J) {
    n2c[J] = mfma16(rN[J], cN[J], zero);
    n2rh[J] = to_h4(mfma16(cN[J], rN[J], zero));
  }
#pragma unroll
  for (int J = 0; J < 4; ++J) {
    n2ch[J] = to_h4(n2c[J]);
    n4c[J] = mfma16(n2rh[J], n2ch[J], zero);
    n4rh[J] = to_h4(mfma16(n2ch[J], n2rh[J], zero));
    p1[J] = to_h4(mfma16(to_h4(n2c[J] + eye), to_h4(eye - rowN[J]), zero));   // row((I - N)(I + N^2))
  }
#pragma unroll
  for (int J = 0; J < 4; ++J) {
    n4ch[J] = to_h4(n4c[J]);
    n8e[J] = to_h4(mfma16(n4rh[J], n4ch[J], zero) + eye);                     // col(I + N^8)
    p2r[J] = to_h4(mfma16(to_h4(n4c[J] + eye), p1[J], zero));                 // row(P1 (I + N^4))
  }
#pragma unroll
  for (int J = 0; J < 4; ++J) {
    Tr[J] = to_h4(mfma16(n8e[J], p2r[J], zero));                              // row(P2 (I + N^8))
    Tc[J] = to_h4(mfma16(p2r[J], n8e[J], zero));                              // col(P2 (I + N^8))
  }
}

// LDS transpose read (ds_read_b64_tr_b16): within each group of 16 lanes, lane i receives
// element (i mod 4) of the 8 bytes addressed by lane (i/4 + 4j), j = 0..3.  frag8_tr builds,
// from a row-major fp16 matrix M[k][m], the fragment in which lane l holds
// M[k0 + 8 (l/16) + e][m0 + l%16], e = 0..7: lane s of a group supplies the addresses of 4
// consecutive columns in rows k0 + 8 (l/16) + s/4 (+4).
typedef short s4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ v4u frag8_tr(const _Float16* base, int ld, int k0, int m0, int lane) {
  const int lr = lane & 15, lg = lane >> 4;
  const _Float16* a = base + (k0 + 8 * lg + (lr >> 2)) * ld + m0 + 4 * (lr & 3);
  typedef unsigned u2 __attribute__((ext_vector_type(2)));
  const u2 x = __builtin_bit_cast(u2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4v*)(a)));
  const u2 y = __builtin_bit_cast(u2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4v*)(a + 4 * ld)));
  return v4u{x[0], x[1], y[0], y[1]};
}
// One transpose read: the accumulator (column) layout of the 16x16 block at (r0, c0) of a
// row-major fp16 matrix, lane l holding M[r0 + 4 (l/16) + e][c0 + l%16], e = 0..3.
__device__ __forceinline__ h4 col_tr(const _Float16* base, int ld, int r0, int c0, int lane) {
  const int lr = lane & 15, lg = lane >> 4;
  const _Float16* a = base + (r0 + 4 * lg + (lr >> 2)) * ld + c0 + 4 * (lr & 3);
  return __builtin_bit_cast(h4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4v*)(a)));
}

// ------------------------------------------------------------------------------------------
// Role: state chain (waves 0, 1).  The wave owns value rows dv = c0 + 16 db + (0..15) and all
// 128 key channels: St[kb] is the accumulator tile (d_k block kb, d_v block db) of S^T, lane
// (lr, lg) holding S[dv = 16 db + lr][dk = 16 kb + 4 lg + e].  Two such tiles regroup in
// registers into the 16x16x32 B operand (contraction over d_k) of X = K S^T; the accumulator
// tiles of X, U and of the decayed U regroup the same way into the B operands of U = T X and of
// the state update, whose A operand K^T comes from the row-major keys through transpose reads.
__device__ __forceinline__ void chain_role(Smem& sm, const ChunkArgs& p, int64_t bh, int c0, int db, int l,
                                           int64_t nchunks) {
  const int lr = l & 15, lg = l >> 4, dv = 16 * db + lr;
  const int64_t T = p.T;
  f4 St[8];
#pragma unroll
  for (int kb = 0; kb < 8; ++kb) {
    f4 x = {0.f, 0.f, 0.f, 0.f};
    if (p.s0) x = *reinterpret_cast<const f4*>(p.s0 + (bh * D + c0 + dv) * D + 16 * kb + 4 * lg);
    St[kb] = x;
  }
  h8 Sb[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    Sb[kk] = pair_k32(to_h4(St[2 * kk]), to_h4(St[2 * kk + 1]));
    *reinterpret_cast<h8*>(&sm.s[dv][32 * kk + 8 * lg]) = Sb[kk];
  }
  __syncthreads();

  for (int64_t c = -2; c < nchunks; ++c) {
    h8 Ud[2];
    float gC = 0.f;
    if (c >= 0) {
      const int b = (int)(c & 1), kb3 = kbuf(c);
      const Gates& g = sm.gt[kb3];
      f4 X[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) X[i] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int i = 0; i < 4; ++i) X[i] = mfma32(lds8(&sm.k[kb3][16 * i + lr][32 * kk + 8 * lg]), Sb[kk], X[i]);
      // lane: tokens 16 i + 4 lg + e, value channel dv
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = 16 * i + 4 * lg;
        const f4 be = *reinterpret_cast<const f4*>(&g.beta[tok]);
        const f4 ga = *reinterpret_cast<const f4*>(&g.gam[tok]);
        const uint2 vv = *reinterpret_cast<const uint2*>(&sm.vt[b][dv][tok]);
        const float v4[4] = {bf16_bits_to_f32(vv.x & 0xffffu), bf16_bits_to_f32(vv.x >> 16),
                             bf16_bits_to_f32(vv.y & 0xffffu), bf16_bits_to_f32(vv.y >> 16)};
#pragma unroll
        for (int e = 0; e < 4; ++e) X[i][e] = be[e] * (v4[e] - ga[e] * X[i][e]);
      }
      const h8 Xb0 = pair_k32(to_h4(X[0]), to_h4(X[1])), Xb1 = pair_k32(to_h4(X[2]), to_h4(X[3]));
      f4 U[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        U[i] = mfma32(lds8(&sm.t[b][16 * i + lr][8 * lg]), Xb0, f4{0.f, 0.f, 0.f, 0.f});
        if (i >= 2) U[i] = mfma32(lds8(&sm.t[b][16 * i + lr][32 + 8 * lg]), Xb1, U[i]);
      }
      *reinterpret_cast<h8*>(&sm.u[dv][8 * lg]) = pair_k32(to_h4(U[0]), to_h4(U[1]));
      *reinterpret_cast<h8*>(&sm.u[dv][32 + 8 * lg]) = pair_k32(to_h4(U[2]), to_h4(U[3]));
#pragma unroll
      for (int i = 0; i < 4; ++i) U[i] *= *reinterpret_cast<const f4*>(&g.dec[16 * i + 4 * lg]);
      Ud[0] = pair_k32(to_h4(U[0]), to_h4(U[1]));
      Ud[1] = pair_k32(to_h4(U[2]), to_h4(U[3]));
      gC = g.gam[C - 1];
    }
    __syncthreads();
    if (c >= 0) {
      const int kb3 = kbuf(c);
      const int64_t t0 = c * C;
      const int n = (int)(T - t0 < C ? T - t0 : C);
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        f4 acc = St[kb] * gC;
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
          acc = mfma32(__builtin_bit_cast(h8, frag8_tr(&sm.k[kb3][0][0], LQ, 32 * kc, 16 * kb, l)), Ud[kc], acc);
        St[kb] = acc;
      }
      if (p.s_ckpt && n == C && ((t0 + n) % p.ckpt_every) == 0) {
        const int64_t idx = (t0 + n) / p.ckpt_every - 1;
        float* dst = p.s_ckpt + ((bh * p.n_ckpt + idx) * D + c0 + dv) * D + 4 * lg;
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) *reinterpret_cast<f4*>(dst + 16 * kb) = St[kb];
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        Sb[kk] = pair_k32(to_h4(St[2 * kk]), to_h4(St[2 * kk + 1]));
        *reinterpret_cast<h8*>(&sm.s[dv][32 * kk + 8 * lg]) = Sb[kk];
      }
    }
    __syncthreads();
  }

  if (p.s_final) {
    float* dst = p.s_final + (bh * D + c0 + dv) * D + 4 * lg;
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) *reinterpret_cast<f4*>(dst + 16 * kb) = St[kb];
  }
}

// ------------------------------------------------------------------------------------------
// Staging.  Global -> registers through buffer loads on per-stream buffer descriptors: the
// hardware range check returns zeros for tokens outside the stream, which pads a ragged last
// chunk with identity steps (k = v = q = 0, beta = 0, log alpha = 0) without branches.  The
// staging roles run branch-free (chunks outside 0..nchunks-1 read as zeros and land in buffers
// nobody reads at that point), so each wait names exactly the loads it needs and the prefetch
// issued in the other phase stays in flight across the barriers (buffer loads never touch the
// LDS counter the barriers wait on).

// Role: outputs of token blocks tb0, tb0 + 1 (waves 4, 5), plus staging of half the queries
// of the next chunk, and of its value slice (wave 4).
// O^T tiles (d_v block d, token block tb): lane holds O[token 16 tb + lr][dv 16 d + 4 lg + e].
// The outputs are written through a buffer descriptor, so rows outside the stream are dropped.
template <typename TOut, int tb0>
__device__ __forceinline__ void out_role(Smem& sm, const ChunkArgs& p, int64_t bh, int c0, int l, int64_t nchunks) {
  constexpr int half = tb0 / 2;
  const int lr = l & 15, lg = l >> 4;
  const int64_t T = p.T, tok0 = bh * T;
  const auto orr = __builtin_amdgcn_make_buffer_rsrc((void*)(static_cast<TOut*>(p.o) + tok0 * D), 0,
                                                     (int)(T * D * (int64_t)sizeof(TOut)), kRsrcWord3);
  const auto qr = stream_rsrc(p.q, tok0 * D, T * D);
  const auto vr = stream_rsrc(p.v, tok0 * D, T * D);
  const int ch = l & 15, rq = l >> 4;   // queries: 16-byte group ch of rows 32 half + 4 i + rq
  const int dq = l & 3, vq = l >> 2;    // values: channels c0 + 8 dq .., tokens 4 vq .. 4 vq + 3
  v4u qv[8], vv[4];
  auto load_q = [&](int64_t t0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) qv[i] = ld_b128(qr, (t0 + 32 * half + 4 * i + rq) * D + 8 * ch);
    if constexpr (half == 0) {
#pragma unroll
      for (int e = 0; e < 4; ++e) vv[e] = ld_b128(vr, (t0 + 4 * vq + e) * D + c0 + 8 * dq);
    }
  };
  load_q(-C);
  __syncthreads();
  for (int64_t c = -2; c < nchunks; ++c) {
    const int b = (int)(c & 1), nb = b ^ 1;
    f4 Oa[2][2];
    // ---- phase 1: O = diag(gamma) Q S^T for chunk c; stage queries (and values) of chunk c + 1
#pragma unroll
    for (int t = 0; t < 2; ++t) Oa[t][0] = Oa[t][1] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      h8 qf[2], sf[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) qf[t] = lds8(&sm.q[b][16 * (tb0 + t) + lr][32 * kk + 8 * lg]);
#pragma unroll
      for (int d = 0; d < 2; ++d) sf[d] = lds8(&sm.s[16 * d + lr][32 * kk + 8 * lg]);
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int d = 0; d < 2; ++d) Oa[t][d] = mfma32(sf[d], qf[t], Oa[t][d]);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const float ga = sm.gt[kbuf(c)].gam[16 * (tb0 + t) + lr];
      Oa[t][0] *= ga;
      Oa[t][1] *= ga;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<h8*>(&sm.q[nb][32 * half + 4 * i + rq][8 * ch]) = bf8_to_h8(qv[i]);
    if constexpr (half == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {  // value channel 8 dq + e: tokens 4 vq .. 4 vq + 3 (bf16 bits)
        uint2 o;
        o.x = pick2(vv[0][e >> 1], vv[1][e >> 1], e);
        o.y = pick2(vv[2][e >> 1], vv[3][e >> 1], e);
        *reinterpret_cast<uint2*>(&sm.vt[nb][8 * dq + e][4 * vq]) = o;
      }
    }
    load_q((c + 2) * C);
    __syncthreads();
    // ---- phase 2: O += P U, write o
    const int64_t t0 = c * C;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int tb = tb0 + t;
#pragma unroll
      for (int kc = 0; kc <= (tb >> 1); ++kc) {  // P is zero above the diagonal blocks
        const h8 pf = lds8(&sm.p[b][16 * tb + lr][32 * kc + 8 * lg]);
#pragma unroll
        for (int d = 0; d < 2; ++d) Oa[t][d] = mfma32(lds8(&sm.u[16 * d + lr][32 * kc + 8 * lg]), pf, Oa[t][d]);
      }
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        const int off = (int)(((t0 + 16 * tb + lr) * D + c0 + 16 * d + 4 * lg) * (int64_t)sizeof(TOut));
        if constexpr (sizeof(TOut) == 2) {
          typedef unsigned u2v __attribute__((ext_vector_type(2)));
          const u2v w = {pack_bf16x2(Oa[t][d][0], Oa[t][d][1]), pack_bf16x2(Oa[t][d][2], Oa[t][d][3])};
          __builtin_amdgcn_raw_buffer_store_b64(w, orr, off, 0, 0);
        } else {
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, Oa[t][d]), orr, off, 0, 0);
        }
      }
    }
    __syncthreads();
  }
}

// Role: diagonal of T (wave 2).  Phase 2 of iteration c forms the diagonal 16x16 blocks of A
// of chunk c + 2 (decay factors, then the key Gram tiles) and stages them on the diagonal of
// T's buffer; phase 1 of the next iteration replaces them by their inverses.
__device__ __forceinline__ void tdiag_role(Smem& sm, int l, int64_t nchunks) {
  const int lr = l & 15, lg = l >> 4;
  __syncthreads();
  for (int64_t c = -2; c < nchunks; ++c) {
    {
      const int nb = (int)((c + 1) & 1);
      f4 rowN[4];
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        const h4 a = lds4(&sm.t[nb][16 * J + lr][16 * J + 4 * lg]);
        rowN[J] = f4{(float)a[0], (float)a[1], (float)a[2], (float)a[3]};
      }
      h4 Tr[4], Tc[4];
      invert_diag4(rowN, lr, lg, Tr, Tc);
#pragma unroll
      for (int J = 0; J < 4; ++J) *reinterpret_cast<h4*>(&sm.t[nb][16 * J + lr][16 * J + 4 * lg]) = Tr[J];
    }
    __syncthreads();
    {
      const int b2 = (int)(c & 1);  // buffer of chunk c + 2
      const Gates& g = sm.gt[kbuf(c + 2)];
      f4 dec[4], acc[4];
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        dec[J] = g.beta[16 * J + lr] * diag_decay(g, J, lr, lg);
        acc[J] = f4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        h8 kf[4];
#pragma unroll
        for (int J = 0; J < 4; ++J) kf[J] = lds8(&sm.k[kbuf(c + 2)][16 * J + lr][32 * kk + 8 * lg]);
#pragma unroll
        for (int J = 0; J < 4; ++J) acc[J] = mfma32(kf[J], kf[J], acc[J]);
      }
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        f4 a = dec[J] * acc[J];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (4 * lg + e == lr) a[e] = 0.f;  // strictly lower
        *reinterpret_cast<h4*>(&sm.t[b2][16 * J + lr][16 * J + 4 * lg]) = to_h4(a);
      }
    }
    __syncthreads();
  }
}

// Role: off-diagonal blocks of T for chunk c + 1 (wave 6, phase 2), by block forward
// substitution down each column, T_ij = T_ii sum_{k=j}^{i-1} (-A_ik) T_kj, in rounds of
// mutually independent blocks: (1,0) (2,1) (3,2), then (2,0) (3,1), then (3,0).  Phase 1
// writes the gate tables of chunk c + 2.
__device__ __forceinline__ void toff_role(Smem& sm, const ChunkArgs& p, int64_t bh, int l, int64_t nchunks) {
  const int lr = l & 15, lg = l >> 4;
  const f4 zero = {0.f, 0.f, 0.f, 0.f};
  const int64_t tok0 = bh * p.T;
  const auto br = stream_rsrc(p.beta, tok0, p.T);
  const auto gr = stream_rsrc(p.log_alpha, tok0, p.T);
  uint32_t bb, gg;
  auto load_g = [&](int64_t t0) {
    bb = __builtin_amdgcn_raw_buffer_load_b16(br, (int)((t0 + l) * 2), 0, 0);
    gg = __builtin_amdgcn_raw_buffer_load_b16(gr, (int)((t0 + l) * 2), 0, 0);
  };
  load_g(0);
  __syncthreads();
  for (int64_t c = -2; c < nchunks; ++c) {
    const int nb = (int)((c + 1) & 1);
    // gate tables of chunk c + 2 (their buffer last held chunk c - 1)
    {
      const float x = wave_prefix_sum(bf16_bits_to_f32(gg & 0xffffu));
      const float glast = __shfl(x, C - 1, 64);
      const float gr1 = __shfl(x, 15, 64), gr2 = __shfl(x, 31, 64), gr3 = __shfl(x, 47, 64);
      const int R = l >> 4;
      const float gref = R == 0 ? 0.f : (R == 1 ? gr1 : (R == 2 ? gr2 : gr3));
      const float beta = bf16_bits_to_f32(bb & 0xffffu);
      Gates& gt = sm.gt[kbuf(c + 2)];
      gt.G[l] = x;
      gt.gam[l] = __expf(x);
      gt.dec[l] = __expf(glast - x);
      gt.beta[l] = beta;
      const float el = __expf(x - gref);
      gt.el[l] = el;
      gt.nbel[l] = -beta * el;
      gt.er[0][l] = __expf(fminf(gr1 - x, 0.f));
      gt.er[1][l] = __expf(fminf(gr2 - x, 0.f));
      gt.er[2][l] = __expf(fminf(gr3 - x, 0.f));
      load_g((c + 3) * C);
    }
    __syncthreads();
    h4 Tr[4], Tc[4], an[6];
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      Tr[J] = lds4(&sm.t[nb][16 * J + lr][16 * J + 4 * lg]);
      Tc[J] = col_tr(&sm.t[nb][0][0], LC, 16 * J, 16 * J, l);
    }
#pragma unroll
    for (int i = 0; i < 6; ++i) an[i] = lds4(&sm.an[i][lr][4 * lg]);
    // lane holds col(T_ij): T[16 i + 4 lg + e][16 j + lr]
    auto put = [&](int i, int j, h4 y) {
#pragma unroll
      for (int e = 0; e < 4; ++e) sm.t[nb][16 * i + 4 * lg + e][16 * j + lr] = y[e];
    };
    h4 y10, y21, y32, y20, y31, y30;
    {
      const h4 z10 = to_h4(mfma16(an[an_idx(1, 0)], Tc[0], zero));
      const h4 z21 = to_h4(mfma16(an[an_idx(2, 1)], Tc[1], zero));
      const h4 z32 = to_h4(mfma16(an[an_idx(3, 2)], Tc[2], zero));
      y10 = to_h4(mfma16(Tr[1], z10, zero));
      y21 = to_h4(mfma16(Tr[2], z21, zero));
      y32 = to_h4(mfma16(Tr[3], z32, zero));
    }
    {
      const h4 z20 = to_h4(mfma16(an[an_idx(2, 1)], y10, mfma16(an[an_idx(2, 0)], Tc[0], zero)));
      const h4 z31 = to_h4(mfma16(an[an_idx(3, 2)], y21, mfma16(an[an_idx(3, 1)], Tc[1], zero)));
      y20 = to_h4(mfma16(Tr[2], z20, zero));
      y31 = to_h4(mfma16(Tr[3], z31, zero));
    }
    {
      const f4 z = mfma16(an[an_idx(3, 1)], y10, mfma16(an[an_idx(3, 0)], Tc[0], zero));
      y30 = to_h4(mfma16(Tr[3], to_h4(mfma16(an[an_idx(3, 2)], y20, z)), zero));
    }
    put(1, 0, y10); put(2, 1, y21); put(3, 2, y32); put(2, 0, y20); put(3, 1, y31); put(3, 0, y30);
    __syncthreads();
  }
}

// Role: keys and P (wave 7).  Phase 1 converts and writes the row-major keys of chunk c + 2
// (their buffer was last read in the previous phase 2); phase 2 computes
// P = tril(Q K^T * D) of chunk c + 1, used by the outputs one iteration later.
__device__ __forceinline__ void pgram_k_role(Smem& sm, const ChunkArgs& p, int64_t bh, int l, int64_t nchunks) {
  const int lr = l & 15, lg = l >> 4;
  constexpr int RR[10] = {0, 1, 2, 3, 1, 2, 3, 2, 3, 3}, JJ[10] = {0, 1, 2, 3, 0, 0, 0, 1, 1, 2};
  const auto kr = stream_rsrc(p.k, bh * p.T * D, p.T * D);
  const int ch = l & 15, rq = l >> 4;   // 16-byte group ch of rows 4 i + rq
  v4u rows[16];
  auto load_rows = [&](int64_t t0) {
#pragma unroll
    for (int i = 0; i < 16; ++i) rows[i] = ld_b128(kr, (t0 + 4 * i + rq) * D + 8 * ch);
  };
  load_rows(0);
  __syncthreads();
  for (int64_t c = -2; c < nchunks; ++c) {
    {
      const int b = kbuf(c + 2);
#pragma unroll
      for (int i = 0; i < 16; ++i) *reinterpret_cast<h8*>(&sm.k[b][4 * i + rq][8 * ch]) = bf8_to_h8(rows[i]);
      load_rows((c + 3) * C);
    }
    __syncthreads();
    const int nb = (int)((c + 1) & 1);
    const Gates& g = sm.gt[kbuf(c + 1)];
    f4 acc[10];
#pragma unroll
    for (int t = 0; t < 10; ++t) acc[t] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      h8 kf[4], qf[4];
#pragma unroll
      for (int J = 0; J < 4; ++J) kf[J] = lds8(&sm.k[kbuf(c + 1)][16 * J + lr][32 * kk + 8 * lg]);
#pragma unroll
      for (int R = 0; R < 4; ++R) qf[R] = lds8(&sm.q[nb][16 * R + lr][32 * kk + 8 * lg]);
#pragma unroll
      for (int t = 0; t < 10; ++t) acc[t] = mfma32(kf[JJ[t]], qf[RR[t]], acc[t]);
    }
#pragma unroll
    for (int J = 0; J < 4; ++J)
      *reinterpret_cast<h4*>(&sm.p[nb][16 * J + lr][16 * J + 4 * lg]) = to_h4(diag_decay(g, J, lr, lg) * acc[J]);
#pragma unroll
    for (int t = 4; t < 10; ++t)
      *reinterpret_cast<h4*>(&sm.p[nb][16 * RR[t] + lr][16 * JJ[t] + 4 * lg]) = to_h4(offdiag_p(g, RR[t], JJ[t], lr, lg, acc[t]));
    __syncthreads();
  }
}

// Role: off-diagonal A (wave 3, phase 1): the off-diagonal blocks of -A of chunk c + 1.
__device__ __forceinline__ void aoff_role(Smem& sm, int l, int64_t nchunks) {
  const int lr = l & 15, lg = l >> 4;
  constexpr int RR[6] = {1, 2, 3, 2, 3, 3}, JJ[6] = {0, 0, 0, 1, 1, 2};
  __syncthreads();
  for (int64_t c = -2; c < nchunks; ++c) {
    const Gates& g = sm.gt[kbuf(c + 1)];
    f4 acc[6];
#pragma unroll
    for (int t = 0; t < 6; ++t) acc[t] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      h8 kf[4];
#pragma unroll
      for (int J = 0; J < 4; ++J) kf[J] = lds8(&sm.k[kbuf(c + 1)][16 * J + lr][32 * kk + 8 * lg]);
#pragma unroll
      for (int t = 0; t < 6; ++t) acc[t] = mfma32(kf[JJ[t]], kf[RR[t]], acc[t]);
    }
#pragma unroll
    for (int t = 0; t < 6; ++t)
      *reinterpret_cast<h4*>(&sm.an[an_idx(RR[t], JJ[t])][lr][4 * lg]) = to_h4(offdiag_neg_a(g, RR[t], JJ[t], lr, lg, acc[t]));
    __syncthreads();
    __syncthreads();
  }
}

template <typename TOut>
__global__ __launch_bounds__(NTH, 1) void gdn_chunk_mfma_kernel(ChunkArgs p) {
  __shared__ Smem sm;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63;

  // XCD-aware placement: consecutive workgroup ids are dealt round-robin over the 8 XCDs;
  // remap so the NT slices of a stream get ids that land on the same XCD.
  const unsigned nblk = gridDim.x;
  unsigned bid = blockIdx.x;
  if (nblk % (8 * NT) == 0) bid = (bid % 8) * (nblk / 8) + bid / 8;
  const int c0 = (int)(bid % NT) * DVT;
  const int64_t bh = bid / NT;
  const int64_t nchunks = (p.T + C - 1) / C;

  // T and P start at zero; their upper blocks are never written
  for (int e = tid; e < 2 * C * LC / 8; e += NTH) reinterpret_cast<v4u*>(&sm.t[0][0][0])[e] = v4u{0u, 0u, 0u, 0u};
  for (int e = tid; e < 2 * C * LC / 8; e += NTH) reinterpret_cast<v4u*>(&sm.p[0][0][0])[e] = v4u{0u, 0u, 0u, 0u};

  // Every role runs nchunks + 2 iterations of two barriers after one initial barrier.  Waves w
  // and w + 4 share a SIMD: the chains (0, 1) share theirs with the outputs (4, 5).
  switch (w) {
    case 0:
    case 1:
      __builtin_amdgcn_s_setprio(2);
      chain_role(sm, p, bh, c0, w, l, nchunks);
      break;
    case 2: tdiag_role(sm, l, nchunks); break;
    case 3: aoff_role(sm, l, nchunks); break;
    case 4: out_role<TOut, 0>(sm, p, bh, c0, l, nchunks); break;
    case 5: out_role<TOut, 2>(sm, p, bh, c0, l, nchunks); break;
    case 6: toff_role(sm, p, bh, l, nchunks); break;
    default: pgram_k_role(sm, p, bh, l, nchunks); break;
  }
}

}  // namespace

bool chunk_mfma_supported(const ChunkArgs& a) {
  // buffer-descriptor offsets are 32-bit: one stream's q/k/v and o must stay under 2 GiB
  return a.in_dtype == GDN_BF16 && a.D == D && a.chunk == C && a.T * D * 4 < (INT64_C(1) << 31);
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
