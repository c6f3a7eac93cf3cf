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
// L2.  Twelve wavefronts take fixed roles (waves w, w + 4 and w + 8 share a SIMD):
//   0, 1    state chain: each keeps a 16 x 128 block of S in fp32 MFMA accumulators for the
//           whole sequence and runs X, U = T X and the state update with every operand
//           regrouped in registers (no LDS round trip on the chunk-to-chunk dependency);
//   4, 5    outputs of two 16-token blocks each, O = diag(gamma) Q S^T + P U, and the keys
//           scaled by e^{G_63 - G} and transposed, the A operand of the state update;
//   10, 11  the causal scores P = tril(Q K^T * D) of the chain's chunk, and the off-diagonal
//           blocks of A two chunks ahead;
//   2, 3    the diagonal 16x16 blocks of A two chunks ahead, and their inverses one ahead;
//   6, 7    keys (fp16, row-major) two chunks ahead, and the off-diagonal blocks of T one ahead;
//   8, 9    gate tables two chunks ahead; queries and the value slice one ahead.
// Each iteration has two barrier-separated phases; the staging waves load from HBM two
// iterations before they store, so global latency never reaches a barrier.
// The products run on v_mfma_f32_16x16x32_f16 / 16x16x16_f16 with fp32 accumulation.
// bf16 inputs convert exactly to fp16 (|x| <= 65504); derived operands (S, P, U, T) are
// rounded to fp16, whose 11-bit significand keeps the bf16-output error budget.
// Layer prologue (optional, template flags): raw gate projections turned into beta and
// log alpha by the gate-table wave; q/k normalisation as per-token factors 1/|k_r|, 1/|q_r|
// computed by the staging waves from the exact fp16 rows and applied where the rows are used
// (Gram tiles, the state chain's beta gamma, the decayed keys, the output rows), so the
// staged tiles stay exact.
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
constexpr int NTH = 768;     // threads per workgroup (12 wavefronts)
constexpr int LQ = D + 16;   // row stride (halves) of [token][channel] tiles: 288 bytes = 72 banks
constexpr int LC = C + 8;    // row stride (halves) of [channel][token] and [token][token] tiles
constexpr int LT = 24;       // row stride (halves) of 16x16 blocks

// Per-chunk gate tables.
struct alignas(16) Gates {
  alignas(16) float G[C];     // inclusive prefix of log alpha
  alignas(16) float gam[C];   // e^{G_r}
  alignas(16) float dec[C];   // e^{G_63 - G_r} / |k_r|
  alignas(16) float beta[C];
  alignas(16) float el[C];    // e^{G_r - G_ref(block of r)}, G_ref(R) = G_{16R-1} (0 for R = 0)
  alignas(16) float nbel[C];  // -beta_r el_r
  alignas(16) float er[3][C]; // er[R-1][j] = e^{G_ref(R) - G_j} for j < 16 R, R = 1..3
  alignas(16) float rk[C];    // 1 / |k_r| when the kernel normalises the keys
  alignas(16) _Float16 bbg[C][2];  // (beta_r, beta_r gamma_r / |k_r|) in fp16, read by the state chain
};

// Buffers hold data of one chunk: keys and gate tables by chunk mod 3, T by chunk mod 2, the
// others single.  Bank layout, as measured on gfx950 with the LDS bank-conflict counter for
// 16-row tiles (lane l on row l%16, 16-byte column chunk l/16): fragment reads are
// conflict-free when the row stride is an odd multiple of 8 four-byte banks, 16-byte writes,
// 8-byte reads and 2-byte writes when it is an odd multiple of 4.  Tiles that are written in
// 16-byte rows and read as fragments (the [token][channel] tiles, the transposed keys, U and P)
// take a stride of the first kind and store the 16-byte chunk c of row r at chunk
// c ^ ((r >> 2) & 1), which makes both conflict-free.  Their rows are always 16 i + l%16 (or
// 4 i + l/16 in the staging stores), so the swizzle costs nothing: it is a per-lane constant.
constexpr int LK = C + 16;   // row stride (halves) of the transposed keys, U and P: 160 bytes = 40 banks
// Swizzled 16-byte chunk l/16 of rows 16 i + l%16, and the same for the 8-byte column groups
// (4 elements) of a 16x16 tile.
__device__ __forceinline__ int swl(int l) { return (l >> 4) ^ ((l >> 2) & 1); }
__device__ __forceinline__ int swl4(int l) { return (l >> 4) ^ (((l >> 2) & 1) << 1); }
struct alignas(16) Smem {
  alignas(16) _Float16 k[3][C][LQ];      // keys                                  [token][d_k]
  alignas(16) _Float16 q[C][LQ];         // queries                               [token][d_k]
  alignas(16) _Float16 s[DVT][LQ];       // fp16 state slice entering the chain's chunk [d_v][d_k]
  alignas(16) _Float16 kt[D][LK];        // keys scaled by e^{G_63 - G}, transposed [d_k][token]
  alignas(16) uint16_t vt[DVT][LC];      // value slice, bf16 bits                [d_v][token]
  alignas(16) _Float16 t[2][C][LC];      // T = (I + A)^{-1}, upper blocks zero; A_JJ staged on the diagonal
  alignas(16) _Float16 p[C][LK];         // tril(Q K^T * D), upper blocks zero     [token][token]
  alignas(16) _Float16 an[2][6][16][LT]; // -A, off-diagonal blocks (R, J), R > J, by chunk mod 2
  alignas(16) _Float16 u[DVT][LK];       // U of the chain's chunk                [d_v][token]
  alignas(16) Gates gt[3];
  alignas(16) float rq[C];               // 1 / |q_r| of the queries' chunk when the kernel normalises them
  alignas(16) float gin[2][2][C];        // raw gates: beta, log alpha of a chunk, activated, by chunk mod 2
};
static_assert(sizeof(Smem) <= 160 * 1024, "LDS budget");
__device__ __forceinline__ int kbuf(int chunk) { return (chunk + 3) % 3; }  // chunk >= -3

constexpr int an_idx(int R, int J) { return R * (R - 1) / 2 + J; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t stream_rsrc(const void* base, int64_t elem0, int64_t n_elems) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)base + elem0), 0, (int)(n_elems * 2), kRsrcWord3);
}
__device__ __forceinline__ v4u ld_b128(__amdgpu_buffer_rsrc_t r, int64_t elem) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)(elem * 2), 0, 0);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ h8 lds8(const _Float16* p) { return *reinterpret_cast<const h8*>(p); }
// Keeps the scheduler from moving instructions across this point: fragment loads for the next
// contraction step are issued before the MFMAs of the current one and no earlier, so at most
// two steps of loads are in flight and each wait names only the step it needs (the LDS counter
// tracks at most 15 outstanding operations).
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }
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

// Inverses of NB unit lower-triangular diagonal blocks (I + N_J), N_J = A_JJ strictly lower,
// as (I - N)(I + N^2)(I + N^4)(I + N^8) (N^16 = 0) on 16x16x16 MFMAs.  With row(M) (lane holds
// M[lr][4lg..+3], the A-operand layout) and col(M) (lane holds M[4lg..+3][lr], the B-operand
// and accumulator layout): col(XY) = mfma(row X, col Y) and row(XY) = mfma(col Y, row X); in
// particular col(N) = mfma(row N, col I).  Returns each inverse in row layout (the factors
// commute, so either order is the product).  The chains are independent and advance level by
// level so their MFMA latencies overlap.
template <int NB>
__device__ __forceinline__ void invert_diag(const f4 (&rowN)[NB], int lr, int lg, h4 (&Tr)[NB]) {
  const f4 zero = {0.f, 0.f, 0.f, 0.f};
  f4 eye;  // identity in either layout: element i of lane (lr, lg) is on the diagonal iff 4 lg + i == lr
#pragma unroll
  for (int i = 0; i < 4; ++i) eye[i] = (4 * lg + i == lr) ? 1.f : 0.f;
  const h4 eyeh = to_h4(eye);
  h4 rN[NB], cN[NB], n2ch[NB], n2rh[NB], n4ch[NB], n4rh[NB], p1[NB], n8e[NB], p2r[NB];
  f4 n2c[NB], n4c[NB];
#pragma unroll
  for (int J = 0; J < NB; ++J) rN[J] = to_h4(rowN[J]);
#pragma unroll
  for (int J = 0; J < NB; ++J) cN[J] = to_h4(mfma16(rN[J], eyeh, zero));
#pragma unroll
  for (int J = 0; J < NB; ++J) {
    n2c[J] = mfma16(rN[J], cN[J], zero);
    n2rh[J] = to_h4(mfma16(cN[J], rN[J], zero));
  }
#pragma unroll
  for (int J = 0; J < NB; ++J) {
    n2ch[J] = to_h4(n2c[J]);
    n4c[J] = mfma16(n2rh[J], n2ch[J], zero);
    n4rh[J] = to_h4(mfma16(n2ch[J], n2rh[J], zero));
    p1[J] = to_h4(mfma16(to_h4(n2c[J] + eye), to_h4(eye - rowN[J]), zero));   // row((I - N)(I + N^2))
  }
#pragma unroll
  for (int J = 0; J < NB; ++J) {
    n4ch[J] = to_h4(n4c[J]);
    n8e[J] = to_h4(mfma16(n4rh[J], n4ch[J], zero) + eye);                     // col(I + N^8)
    p2r[J] = to_h4(mfma16(to_h4(n4c[J] + eye), p1[J], zero));                 // row(P1 (I + N^4))
  }
#pragma unroll
  for (int J = 0; J < NB; ++J) Tr[J] = to_h4(mfma16(n8e[J], p2r[J], zero));   // row(P2 (I + N^8))
}

// LDS transpose read (ds_read_b64_tr_b16): within each group of 16 lanes, lane i receives
// element (i mod 4) of the 8 bytes addressed by lane (i/4 + 4j), j = 0..3.  frag8_tr builds,
// from a row-major fp16 matrix M[k][m], the fragment in which lane l holds
// M[k0 + 8 (l/16) + e][m0 + l%16], e = 0..7: lane s of a group supplies the addresses of 4
// consecutive columns in rows k0 + 8 (l/16) + s/4 (+4) of a chunk-swizzled tile (k0 a
// multiple of 32, m0 of 16).
typedef short s4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ v4u frag8_tr(const _Float16* base, int ld, int k0, int m0, int lane) {
  const int lr = lane & 15, lg = lane >> 4;
  const _Float16* a = base + (k0 + 8 * lg + (lr >> 2)) * ld + m0 + 4 * (lr & 3);
  typedef unsigned u2 __attribute__((ext_vector_type(2)));
  const u2 x = __builtin_bit_cast(u2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4v*)(a)));
  // rows k0 + 8 (l/16) + 4 + s/4 have bit 2 set: their 16-byte chunks are swapped in pairs
  const _Float16* b = base + (k0 + 8 * lg + (lr >> 2) + 4) * ld + m0 + ((4 * (lr & 3)) ^ 8);
  const u2 y = __builtin_bit_cast(u2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4v*)(b)));
  return v4u{x[0], x[1], y[0], y[1]};
}
// One transpose read: the accumulator (column) layout of the 16x16 block at (r0, c0) of a
// row-major fp16 matrix, lane l holding M[r0 + 4 (l/16) + e][c0 + l%16], e = 0..3.
__device__ __forceinline__ h4 col_tr(const _Float16* base, int ld, int r0, int c0, int lane) {
  const int lr = lane & 15, lg = lane >> 4;
  const _Float16* a = base + (r0 + 4 * lg + (lr >> 2)) * ld + c0 + 4 * (lr & 3);
  return __builtin_bit_cast(h4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4v*)(a)));
}

// Where one (sequence, value head) stream lives: its token count, the element offset of its
// rows in q and k, the token offset of its rows in v, o and of its gates, and the index of its
// states in s0, s_final and s_ckpt.  A batch of equal-length sequences is [B, H(qk), T, D]; a
// ragged batch concatenates the sequences, each in that layout with its own length.
struct Stream {
  int64_t T, qk, tok, st;
};

// ------------------------------------------------------------------------------------------
// Role: state chain (waves 0, 1).  The wave owns value rows dv = c0 + 16 db + (0..15) and all
// 128 key channels: St[kb] is the accumulator tile (d_k block kb, d_v block db) of S^T, lane
// (lr, lg) holding S[dv = 16 db + lr][dk = 16 kb + 4 lg + e].  Two such tiles regroup in
// registers into the 16x16x32 B operand (contraction over d_k) of X = K S^T; the accumulator
// tiles of X and U regroup the same way into the B operands of U = T X and of the state update
// S^T <- gamma_63 S^T + (diag(e^{G_63 - G}) K)^T U.  Its A operand, the decayed transposed keys,
// is staged by the output waves in two halves: tokens 0..31 one phase ahead (fetched with the
// other phase-1 operands) and tokens 32..63 in phase 1 (fetched at the start of phase 2).
__device__ __forceinline__ void chain_role(Smem& sm, const ChunkArgs& p, const Stream& str, int c0, int db, int l,
                                           int64_t nchunks) {
  const int lr = l & 15, lg = l >> 4, dv = 16 * db + lr, sg = swl(l);
  const int64_t T = str.T, bh = str.st;
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
    *reinterpret_cast<h8*>(&sm.s[dv][32 * kk + 8 * sg]) = Sb[kk];
  }
  __syncthreads();

  for (int c = -2; c < (int)nchunks; ++c) {
    h8 Ub[2], kt0[8];
    if (c >= 0) {
      const int kb3 = kbuf(c);
      const Gates& g = sm.gt[kb3];
      h8 bg[4];    // (beta, beta gamma) of tokens 16 i + 4 lg + e
      uint2 vv[4]; // values of those tokens, bf16
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bg[i] = lds8(&g.bbg[16 * i + 4 * lg][0]);
        vv[i] = *reinterpret_cast<const uint2*>(&sm.vt[dv][16 * i + 4 * lg]);
      }
      f4 X[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) X[i] = f4{0.f, 0.f, 0.f, 0.f};
      h8 kfr[2][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) kfr[0][i] = lds8(&sm.k[kb3][16 * i + lr][8 * sg]);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        if (kk < 3) {
#pragma unroll
          for (int i = 0; i < 4; ++i) kfr[(kk + 1) & 1][i] = lds8(&sm.k[kb3][16 * i + lr][32 * (kk + 1) + 8 * sg]);
        }
        sched_fence();
#pragma unroll
        for (int i = 0; i < 4; ++i) X[i] = mfma32(kfr[kk & 1][i], Sb[kk], X[i]);
        sched_fence();
      }
      h8 tf[6];
#pragma unroll
      for (int i = 0, m = 0; i < 4; ++i) {
        tf[m++] = lds8(&sm.t[(int)(c & 1)][16 * i + lr][8 * lg]);
        if (i >= 2) tf[m++] = lds8(&sm.t[(int)(c & 1)][16 * i + lr][32 + 8 * lg]);
      }
      // lane: tokens 16 i + 4 lg + e, value channel dv; X = beta v - beta gamma (K S^T)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v4[4] = {bf16_bits_to_f32(vv[i].x & 0xffffu), bf16_bits_to_f32(vv[i].x >> 16),
                             bf16_bits_to_f32(vv[i].y & 0xffffu), bf16_bits_to_f32(vv[i].y >> 16)};
#pragma unroll
        for (int e = 0; e < 4; ++e) X[i][e] = (float)bg[i][2 * e] * v4[e] - (float)bg[i][2 * e + 1] * X[i][e];
      }
      const h8 Xb0 = pair_k32(to_h4(X[0]), to_h4(X[1])), Xb1 = pair_k32(to_h4(X[2]), to_h4(X[3]));
      f4 U[4];
#pragma unroll
      for (int i = 0, m = 0; i < 4; ++i) {
        U[i] = mfma32(tf[m++], Xb0, f4{0.f, 0.f, 0.f, 0.f});
        if (i >= 2) U[i] = mfma32(tf[m++], Xb1, U[i]);
      }
      Ub[0] = pair_k32(to_h4(U[0]), to_h4(U[1]));
      Ub[1] = pair_k32(to_h4(U[2]), to_h4(U[3]));
      *reinterpret_cast<h8*>(&sm.u[dv][8 * sg]) = Ub[0];
      *reinterpret_cast<h8*>(&sm.u[dv][32 + 8 * sg]) = Ub[1];
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) kt0[kb] = lds8(&sm.kt[16 * kb + lr][8 * sg]);
      const float gC = g.gam[C - 1];
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) St[kb] *= gC;
    }
    __syncthreads();
    if (c >= 0) {
      const int64_t t0 = (int64_t)c * C;
      const int n = (int)(T - t0 < C ? T - t0 : C);
      h8 kt1[8];
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) kt1[kb] = lds8(&sm.kt[16 * kb + lr][32 + 8 * sg]);
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) St[kb] = mfma32(kt1[kb], Ub[1], mfma32(kt0[kb], Ub[0], St[kb]));
      if (p.s_ckpt && n == C && ((t0 + n) % p.ckpt_every) == 0) {
        const int64_t idx = (t0 + n) / p.ckpt_every - 1;
        float* dst = p.s_ckpt + ((bh * p.n_ckpt + idx) * D + c0 + dv) * D + 4 * lg;
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) *reinterpret_cast<f4*>(dst + 16 * kb) = St[kb];
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        Sb[kk] = pair_k32(to_h4(St[2 * kk]), to_h4(St[2 * kk + 1]));
        *reinterpret_cast<h8*>(&sm.s[dv][32 * kk + 8 * sg]) = Sb[kk];
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

// Value of x in the partner lane of a DPP row permutation: row_mirror (0x140, lane c of the
// 16-lane row reads lane 15 - c), row_half_mirror (0x141, 7 - c within each half row),
// quad_perm 2,3,0,1 (0x4e, c ^ 2) and quad_perm 1,0,3,2 (0xb1, c ^ 1).
template <int CTRL>
__device__ __forceinline__ float dpp_partner(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}
// Reduce-scatter of eight per-lane partial sums ss[i] over the 16 lanes of a DPP row: each
// exchange pairs lanes from different halves of the set of lanes already summed and keeps half
// of the rows, so 4 + 2 + 1 + 1 exchanges replace 8 x 4.  Lane c ends with the full sum of row
// 4 [c >= 8] + 2 [c % 8 >= 4] + [c & 2] (lanes c and c ^ 1 hold the same row); returns it and
// the row index.
__device__ __forceinline__ float row16_reduce_scatter(const float (&ss)[8], int c, int& row) {
  const bool hA = c >= 8, hB = (c & 7) >= 4, hC = (c & 2) != 0;
  float a[4], b[2];
#pragma unroll
  for (int j = 0; j < 4; ++j) a[j] = (hA ? ss[j + 4] : ss[j]) + dpp_partner<0x140>(hA ? ss[j] : ss[j + 4]);
#pragma unroll
  for (int m = 0; m < 2; ++m) b[m] = (hB ? a[m + 2] : a[m]) + dpp_partner<0x141>(hB ? a[m] : a[m + 2]);
  const float x = (hC ? b[1] : b[0]) + dpp_partner<0x4e>(hC ? b[0] : b[1]);
  row = 4 * hA + 2 * hB + hC;
  return x + dpp_partner<0xb1>(x);
}

// Half of the row-major tokens of a chunk (rows 32 half + 0..31) of a [token][d_k] bf16 input,
// converted to fp16 into a chunk-swizzled LDS tile (row 32 half + 4 i + rq has bit 2 = i & 1).
// With L2N the tile keeps the rows as given and rn[row] receives 1 / sqrt(sum(x^2) + 1e-6),
// the factor that scales the row to unit length ("Attention, Part 4", section 6: queries and
// keys are normalised before the memory step); the consumers apply it per token.  The 16
// lanes of a row form one DPP row; the squares of the exact fp16 values sum in fp32.
template <int half, bool L2N>
struct RowStage {
  __amdgpu_buffer_rsrc_t r;
  v4u x[8];
  int ch, rq;
  __device__ __forceinline__ RowStage(const void* base, const Stream& str, int l)
      : r(stream_rsrc(base, str.qk, str.T * D)), ch(l & 15), rq(l >> 4) {}
  __device__ __forceinline__ void load(int64_t t0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = ld_b128(r, (t0 + 32 * half + 4 * i + rq) * D + 8 * ch);
  }
  __device__ __forceinline__ void store(_Float16 (*dst)[LQ], float* rn) const {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    float ss[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const h8 y = bf8_to_h8(x[i]);
      *reinterpret_cast<h8*>(&dst[32 * half + 4 * i + rq][8 * (ch ^ (i & 1))]) = y;
      if constexpr (L2N) {
        ss[i] = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const h2 pr = {y[2 * e], y[2 * e + 1]};
          ss[i] = __builtin_amdgcn_fdot2(pr, pr, ss[i], false);
        }
      }
    }
    if constexpr (L2N) {  // row 4 i + rq of the half: the two lanes holding row i write the same value
      int i;
      const float sum = row16_reduce_scatter(ss, ch, i);
      rn[32 * half + 4 * i + rq] = __builtin_amdgcn_rsqf(sum + 1e-6f);  // argument >= 1e-6: no denormal
    }
  }
  // The row factors alone, from the registers (the same arithmetic as store).
  __device__ __forceinline__ void norms(float* rn) const {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    float ss[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const h8 y = bf8_to_h8(x[i]);
      ss[i] = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const h2 pr = {y[2 * e], y[2 * e + 1]};
        ss[i] = __builtin_amdgcn_fdot2(pr, pr, ss[i], false);
      }
    }
    int i;
    const float sum = row16_reduce_scatter(ss, ch, i);
    rn[32 * half + 4 * i + rq] = __builtin_amdgcn_rsqf(sum + 1e-6f);
  }
};

// Decayed, transposed keys for 4 d_k blocks kb0.. and one 32-token half kc of a chunk: transpose
// reads from the row-major keys, each token scaled by e^{G_63 - G}.
__device__ __forceinline__ void stage_kt(Smem& sm, const _Float16* k, const Gates& g, int kb0, int kc, int l) {
  const int lr = l & 15, lg = l >> 4, sg = swl(l);
  const h4 a = to_h4(*reinterpret_cast<const f4*>(&g.dec[32 * kc + 8 * lg]));
  const h4 b = to_h4(*reinterpret_cast<const f4*>(&g.dec[32 * kc + 8 * lg + 4]));
  const h8 dech = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int dk0 = 16 * (kb0 + j);
    const h8 x = __builtin_bit_cast(h8, frag8_tr(k, LQ, 32 * kc, dk0, l)) * dech;
    *reinterpret_cast<h8*>(&sm.kt[dk0 + lr][32 * kc + 8 * sg]) = x;
  }
}

// Role: outputs of token blocks tb0, tb0 + 1 (waves 4, 5).  O^T tiles (d_v block d, token block
// tb): lane holds O[token 16 tb + lr][dv 16 d + 4 lg + e], written through a buffer descriptor
// so rows outside the stream are dropped.  The wave also stages the decayed transposed keys of
// d_k blocks 2 tb0 .. 2 tb0 + 3: tokens 32..63 of chunk c in phase 1 and tokens 0..31 of chunk
// c + 1 in phase 2 (each half is read by the chain in the phase after it is written).
template <typename TOut, int tb0, bool L2N>
__device__ __forceinline__ void out_role(Smem& sm, const ChunkArgs& p, const Stream& str, int c0, int l,
                                         int64_t nchunks) {
  const int lr = l & 15, lg = l >> 4, sg = swl(l);
  const int64_t T = str.T, tok0 = str.tok;
  const auto orr = __builtin_amdgcn_make_buffer_rsrc((void*)(static_cast<TOut*>(p.o) + tok0 * D), 0,
                                                     (int)(T * D * (int64_t)sizeof(TOut)), kRsrcWord3);
  __syncthreads();
  for (int c = -2; c < (int)nchunks; ++c) {
    f4 Oa[2][2];
    // ---- phase 1: O = diag(gamma) Q S^T for chunk c
#pragma unroll
    for (int t = 0; t < 2; ++t) Oa[t][0] = Oa[t][1] = f4{0.f, 0.f, 0.f, 0.f};
    {
      h8 fr[2][4];  // [step parity][q0 q1 s0 s1]
      auto ld = [&](int kk, h8 (&f)[4]) {
#pragma unroll
        for (int t = 0; t < 2; ++t) f[t] = lds8(&sm.q[16 * (tb0 + t) + lr][32 * kk + 8 * sg]);
#pragma unroll
        for (int d = 0; d < 2; ++d) f[2 + d] = lds8(&sm.s[16 * d + lr][32 * kk + 8 * sg]);
      };
      ld(0, fr[0]);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        if (kk < 3) ld(kk + 1, fr[(kk + 1) & 1]);
        sched_fence();
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int d = 0; d < 2; ++d) Oa[t][d] = mfma32(fr[kk & 1][2 + d], fr[kk & 1][t], Oa[t][d]);
        sched_fence();
      }
    }
    float rqv[2];  // 1 / |q| of the lane's two output rows (the queries' buffer is refilled in phase 2)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const float ga = sm.gt[kbuf(c)].gam[16 * (tb0 + t) + lr];
      Oa[t][0] *= ga;
      Oa[t][1] *= ga;
      rqv[t] = L2N ? sm.rq[16 * (tb0 + t) + lr] : 1.f;
    }
    stage_kt(sm, &sm.k[kbuf(c)][0][0], sm.gt[kbuf(c)], 2 * tb0, 1, l);
    __syncthreads();
    // ---- phase 2: O += P U, write o; transposed keys (tokens 0..31) of chunk c + 1
    const int64_t t0 = (int64_t)c * C;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int tb = tb0 + t;
#pragma unroll
      for (int kc = 0; kc <= (tb >> 1); ++kc) {  // P is zero above the diagonal blocks
        const h8 pf = lds8(&sm.p[16 * tb + lr][32 * kc + 8 * sg]);
#pragma unroll
        for (int d = 0; d < 2; ++d) Oa[t][d] = mfma32(lds8(&sm.u[16 * d + lr][32 * kc + 8 * sg]), pf, Oa[t][d]);
      }
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        if constexpr (L2N) Oa[t][d] *= rqv[t];  // both terms of the output row carry 1 / |q_r|
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
    stage_kt(sm, &sm.k[kbuf(c + 1)][0][0], sm.gt[kbuf(c + 1)], 2 * tb0, 0, l);
    __syncthreads();
  }
}

// Role: diagonal of T, blocks J0 and J0 + 1 (waves 2, 3).  Phase 2 of iteration c forms the
// diagonal 16x16 blocks of A of chunk c + 2 (decay factors, then the key Gram tiles) and stages
// them on the diagonal of T's buffer; phase 1 of the next iteration replaces them by their
// inverses.
template <int J0, bool L2N>
__device__ __forceinline__ void tdiag_role(Smem& sm, int l, int64_t nchunks) {
  const int lr = l & 15, lg = l >> 4;
  __syncthreads();
  for (int c = -2; c < (int)nchunks; ++c) {
    {
      const int nb = (int)((c + 1) & 1);
      f4 rowN[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const h4 a = lds4(&sm.t[nb][16 * (J0 + j) + lr][16 * (J0 + j) + 4 * lg]);
        rowN[j] = f4{(float)a[0], (float)a[1], (float)a[2], (float)a[3]};
      }
      h4 Tr[2];
      invert_diag<2>(rowN, lr, lg, Tr);
#pragma unroll
      for (int j = 0; j < 2; ++j) *reinterpret_cast<h4*>(&sm.t[nb][16 * (J0 + j) + lr][16 * (J0 + j) + 4 * lg]) = Tr[j];
    }
    __syncthreads();
    {
      const int b2 = (int)(c & 1);  // T buffer of chunk c + 2
      const Gates& g = sm.gt[kbuf(c + 2)];
      f4 dec[2], acc[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        dec[j] = g.beta[16 * (J0 + j) + lr] * diag_decay(g, J0 + j, lr, lg);
        acc[j] = f4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const h8 kf = lds8(&sm.k[kbuf(c + 2)][16 * (J0 + j) + lr][32 * kk + 8 * swl(l)]);
          acc[j] = mfma32(kf, kf, acc[j]);
        }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if constexpr (L2N)  // unit keys: rows and columns of K K^T scale by 1 / |k|
          dec[j] *= g.rk[16 * (J0 + j) + lr] * *reinterpret_cast<const f4*>(&g.rk[16 * (J0 + j) + 4 * lg]);
        f4 a = dec[j] * acc[j];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (4 * lg + e == lr) a[e] = 0.f;  // strictly lower
        *reinterpret_cast<h4*>(&sm.t[b2][16 * (J0 + j) + lr][16 * (J0 + j) + 4 * lg]) = to_h4(a);
      }
    }
    __syncthreads();
  }
}

// Off-diagonal blocks of T for chunk c + 1 by block forward substitution down a column,
// T_ij = T_ii sum_{k=j}^{i-1} (-A_ik) T_kj; lane holds col(T_ij): T[16 i + 4 lg + e][16 j + lr].
// COLS = 0: column 0 (blocks (1,0), (2,0), (3,0)); COLS = 1: columns 1 and 2.
template <int COLS>
__device__ __forceinline__ void toff_part(Smem& sm, int64_t c, int l) {
  const int lr = l & 15, lg = l >> 4;
  const f4 zero = {0.f, 0.f, 0.f, 0.f};
  const int nb = (int)((c + 1) & 1);
  auto tr = [&](int i) { return lds4(&sm.t[nb][16 * i + lr][16 * i + 4 * lg]); };
  auto an = [&](int i, int k) { return lds4(&sm.an[nb][an_idx(i, k)][lr][4 * lg]); };
  auto put = [&](int i, int j, h4 y) {
#pragma unroll
    for (int e = 0; e < 4; ++e) sm.t[nb][16 * i + 4 * lg + e][16 * j + lr] = y[e];
  };
  if constexpr (COLS == 0) {
    const h4 tc0 = col_tr(&sm.t[nb][0][0], LC, 0, 0, l);
    const h4 t1 = tr(1), t2 = tr(2), t3 = tr(3);
    const h4 a10 = an(1, 0), a20 = an(2, 0), a21 = an(2, 1), a30 = an(3, 0), a31 = an(3, 1), a32 = an(3, 2);
    const f4 p20 = mfma16(a20, tc0, zero), p30 = mfma16(a30, tc0, zero);
    const h4 y10 = to_h4(mfma16(t1, to_h4(mfma16(a10, tc0, zero)), zero));
    const h4 y20 = to_h4(mfma16(t2, to_h4(mfma16(a21, y10, p20)), zero));
    const h4 y30 = to_h4(mfma16(t3, to_h4(mfma16(a32, y20, mfma16(a31, y10, p30))), zero));
    put(1, 0, y10); put(2, 0, y20); put(3, 0, y30);
  } else {
    const h4 tc1 = col_tr(&sm.t[nb][0][0], LC, 16, 16, l), tc2 = col_tr(&sm.t[nb][0][0], LC, 32, 32, l);
    const h4 t2 = tr(2), t3 = tr(3);
    const h4 a21 = an(2, 1), a31 = an(3, 1), a32 = an(3, 2);
    const f4 p31 = mfma16(a31, tc1, zero);
    const h4 y21 = to_h4(mfma16(t2, to_h4(mfma16(a21, tc1, zero)), zero));
    const h4 y32 = to_h4(mfma16(t3, to_h4(mfma16(a32, tc2, zero)), zero));
    const h4 y31 = to_h4(mfma16(t3, to_h4(mfma16(a32, y21, p31)), zero));
    put(2, 1, y21); put(3, 2, y32); put(3, 1, y31);
  }
}

// Role: keys of chunk c + 2, half `half` (waves 6, 7, phase 1; their buffer was last read in the
// previous phase 2), and part COLS = half of the off-diagonal blocks of T for chunk c + 1
// (phase 2).
template <int half, bool L2N>
__device__ __forceinline__ void key_toff_role(Smem& sm, const ChunkArgs& p, const Stream& str, int l,
                                              int64_t nchunks) {
  // two register sets: each chunk's rows are loaded two iterations before they are stored
  RowStage<half, L2N> ka(p.k, str, l), kb(p.k, str, l);
  // wave 7, with q normalisation: the norms of the second half of the queries of chunk c + 1
  // (phase 2), from rows loaded one iteration before
  constexpr bool QN = L2N && half == 1;
  RowStage<1, false> q2(p.q, str, l);
  ka.load(0);
  kb.load(C);
  if constexpr (QN) q2.load(-C);
  auto iter = [&](int c, RowStage<half, L2N>& ks) {
    ks.store(sm.k[kbuf(c + 2)], sm.gt[kbuf(c + 2)].rk);
    ks.load((int64_t)(c + 4) * C);
    __syncthreads();
    toff_part<half>(sm, c, l);
    if constexpr (QN) {
      q2.norms(sm.rq);
      q2.load((int64_t)(c + 2) * C);
    }
    __syncthreads();
  };
  __syncthreads();
  for (int c = -2; c < (int)nchunks; c += 2) {
    iter(c, ka);
    if (c + 1 < (int)nchunks) iter(c + 1, kb);
  }
}

// Role: gate tables of chunk c + 2 (wave 8, phase 1; their buffer last held chunk c - 1), and the
// second half of the queries and the value slice of chunk c + 1 (phase 2; every reader of those
// buffers runs in phase 1).
template <bool RAW, bool L2N>
__device__ __forceinline__ void gates_qv_role(Smem& sm, const ChunkArgs& p, const Stream& str, int c0, int l,
                                              int64_t nchunks) {
  const int64_t tok0 = str.tok, T = str.T;
  const auto br = stream_rsrc(p.beta, tok0, T);
  const auto gr = stream_rsrc(p.log_alpha, tok0, T);
  const auto vr = stream_rsrc(p.v, tok0 * D, T * D);
  // values: channels c0 + 8 dq .., tokens 4 vq .. 4 vq + 3; with the 16 token groups on
  // consecutive lanes the transposed 8-byte stores are free of LDS bank conflicts
  const int dq = l >> 4, vq = l & 15;
  struct Set {
    uint32_t bb, gg;
    v4u vv[4];
  };
  RowStage<1, false> qa(p.q, str, l), qb(p.q, str, l);  // their norms come from wave 7
  Set sa, sb;
  auto load_g = [&](Set& st, int64_t t0) {
    if constexpr (RAW) return;  // raw gates arrive activated, through sm.gin
    st.bb = __builtin_amdgcn_raw_buffer_load_b16(br, (int)((t0 + l) * 2), 0, 0);
    st.gg = __builtin_amdgcn_raw_buffer_load_b16(gr, (int)((t0 + l) * 2), 0, 0);
  };
  auto load_v = [&](Set& st, int64_t t0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) st.vv[e] = ld_b128(vr, (t0 + 4 * vq + e) * D + c0 + 8 * dq);
  };
  // two register sets: gates of chunk c + 2 and queries/values of chunk c + 1 are loaded two
  // iterations before they are stored
  load_g(sa, 0);
  load_g(sb, C);
  qa.load(-C);
  load_v(sa, -C);
  qb.load(0);
  load_v(sb, 0);
  auto iter = [&](int c, Set& st, RowStage<1, false>& qs) {
    float dl, bgam;  // e^{G_63 - G_l} and beta gamma of chunk c + 2, scaled by 1 / |k_l| in phase 2 with L2N
    {
      float g, bt;
      if constexpr (RAW) {  // activated by the query wave one iteration ago
        bt = sm.gin[(c + 2) & 1][0][l];
        g = sm.gin[(c + 2) & 1][1][l];
      } else {
        g = bf16_bits_to_f32(st.gg & 0xffffu);
        bt = bf16_bits_to_f32(st.bb & 0xffffu);
      }
      const float x = wave_prefix_sum(g);
      const float glast = __shfl(x, C - 1, 64);
      const float gr1 = __shfl(x, 15, 64), gr2 = __shfl(x, 31, 64), gr3 = __shfl(x, 47, 64);
      const int R = l >> 4;
      const float gref = R == 0 ? 0.f : (R == 1 ? gr1 : (R == 2 ? gr2 : gr3));
      const float beta = bt;
      Gates& gt = sm.gt[kbuf(c + 2)];
      const float gam = __expf(x), el = __expf(x - gref);
      gt.G[l] = x;
      gt.gam[l] = gam;
      dl = __expf(glast - x);
      bgam = beta * gam;
      if constexpr (!L2N) gt.dec[l] = dl;
      gt.beta[l] = beta;
      gt.el[l] = el;
      gt.nbel[l] = -beta * el;
      gt.er[0][l] = __expf(fminf(gr1 - x, 0.f));
      gt.er[1][l] = __expf(fminf(gr2 - x, 0.f));
      gt.er[2][l] = __expf(fminf(gr3 - x, 0.f));
      gt.bbg[l][0] = (_Float16)beta;
      if constexpr (!L2N) gt.bbg[l][1] = (_Float16)bgam;
      load_g(st, (int64_t)(c + 4) * C);
    }
    __syncthreads();
    qs.store(sm.q, nullptr);
    qs.load((int64_t)(c + 3) * C);
    if constexpr (L2N) {  // the key norms of chunk c + 2 were staged in phase 1
      Gates& gt = sm.gt[kbuf(c + 2)];
      const float r = gt.rk[l];
      gt.dec[l] = dl * r;
      gt.bbg[l][1] = (_Float16)(bgam * r);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {  // value channel 8 dq + e: tokens 4 vq .. 4 vq + 3 (bf16 bits)
      uint2 o;
      o.x = pick2(st.vv[0][e >> 1], st.vv[1][e >> 1], e);
      o.y = pick2(st.vv[2][e >> 1], st.vv[3][e >> 1], e);
      *reinterpret_cast<uint2*>(&sm.vt[8 * dq + e][4 * vq]) = o;
    }
    load_v(st, (int64_t)(c + 3) * C);
    __syncthreads();
  };
  __syncthreads();
  for (int c = -2; c < (int)nchunks; c += 2) {
    iter(c, sa, qa);
    if (c + 1 < (int)nchunks) iter(c + 1, sb, qb);
  }
}

// Role: first half of the queries of chunk c + 1 (wave 9, phase 2), loaded two iterations ahead.
// With raw gates, phase 1 (otherwise idle) takes the gate activations off the gates wave:
// beta = sigmoid(b) and log alpha = -exp(A_log) softplus(a + dt_bias) of chunk c + 3 ("Attention,
// Part 4", section "Where alpha and beta come from"), into sm.gin (by chunk mod 2) for the gates
// wave's next iteration; b and a are loaded one iteration before.  Tokens past the end read as
// b = a = 0 and must stay identity steps, so they take beta = log alpha = 0.
template <bool RAW, bool L2N>
__device__ __forceinline__ void q_role(Smem& sm, const ChunkArgs& p, const Stream& str, int l, int64_t nchunks) {
  RowStage<0, L2N> qa(p.q, str, l), qb(p.q, str, l);
  qa.load(-C);
  qb.load(0);
  const int64_t T = str.T;
  const auto br = stream_rsrc(p.beta, str.tok, T);
  const auto gr = stream_rsrc(p.log_alpha, str.tok, T);
  float Aexp = 0.f, dtb = 0.f;
  uint32_t bb = 0, gg = 0;
  auto load_g = [&](int chunk) {
    bb = __builtin_amdgcn_raw_buffer_load_b16(br, (int)(((int64_t)chunk * C + l) * 2), 0, 0);
    gg = __builtin_amdgcn_raw_buffer_load_b16(gr, (int)(((int64_t)chunk * C + l) * 2), 0, 0);
  };
  auto activate = [&](int chunk) {
    const bool live = (int64_t)chunk * C + l < T;
    float g = bf16_bits_to_f32(gg & 0xffffu), bt = bf16_bits_to_f32(bb & 0xffffu);
    const float xa = g + dtb;
    g = live ? -Aexp * (fmaxf(xa, 0.f) + log1pf(__expf(-fabsf(xa)))) : 0.f;  // softplus, no overflow
    bt = live ? 1.f / (1.f + __expf(-bt)) : 0.f;
    sm.gin[chunk & 1][0][l] = bt;
    sm.gin[chunk & 1][1][l] = g;
  };
  if constexpr (RAW) {
    const int64_t h = str.st % p.H;
    Aexp = __expf(p.A_log[h]);
    dtb = p.dt_bias[h];
    load_g(0);
    activate(0);  // read by the gates wave in the first iteration
    load_g(1);
  }
  auto iter = [&](int c, RowStage<0, L2N>& qs) {
    if constexpr (RAW) {
      activate(c + 3);
      load_g(c + 4);
    }
    __syncthreads();
    qs.store(sm.q, sm.rq);
    qs.load((int64_t)(c + 3) * C);
    __syncthreads();
  };
  __syncthreads();
  for (int c = -2; c < (int)nchunks; c += 2) {
    iter(c, qa);
    if (c + 1 < (int)nchunks) iter(c + 1, qb);
  }
}

// Role: half SET of the tiles of P = tril(Q K^T * D) of chunk c (waves 10, 11, phase 1; read by
// the outputs in phase 2), and half SET of the off-diagonal blocks of -A of chunk c + 2
// (phase 2; their keys and gates were staged in phase 1), used one iteration later.
template <int SET, bool L2N>
__device__ __forceinline__ void pa_role(Smem& sm, int l, int64_t nchunks) {
  const int lr = l & 15, lg = l >> 4;
  // P tiles (R, J): set 0 = (0,0) (1,1) (1,0) (2,0) (3,0); set 1 = (2,2) (3,3) (2,1) (3,1) (3,2).
  constexpr int PR[2][5] = {{0, 1, 1, 2, 3}, {2, 3, 2, 3, 3}}, PJ[2][5] = {{0, 1, 0, 0, 0}, {2, 3, 1, 1, 2}};
  // A tiles: set 0 = (1,0) (2,0) (3,0); set 1 = (2,1) (3,1) (3,2).
  constexpr int AR[2][3] = {{1, 2, 3}, {2, 3, 3}}, AJ[2][3] = {{0, 0, 0}, {1, 1, 2}};
  constexpr int J0 = SET == 0 ? 0 : 1, J1 = SET == 0 ? 1 : 3;   // key blocks of P's tiles
  constexpr int R0 = SET == 0 ? 0 : 2;                           // query blocks R0..3
  __syncthreads();
  for (int c = -2; c < (int)nchunks; ++c) {
    {
      const Gates& g = sm.gt[kbuf(c)];
      f4 fac[5], acc[5], rkc[5];
#pragma unroll
      for (int t = 0; t < 5; ++t) acc[t] = f4{0.f, 0.f, 0.f, 0.f};
      {
        h8 kf[2][4], qf[2][4];
        auto ld = [&](int kk, h8 (&k4)[4], h8 (&q4)[4]) {
#pragma unroll
          for (int J = J0; J <= J1; ++J) k4[J] = lds8(&sm.k[kbuf(c)][16 * J + lr][32 * kk + 8 * swl(l)]);
#pragma unroll
          for (int R = R0; R < 4; ++R) q4[R] = lds8(&sm.q[16 * R + lr][32 * kk + 8 * swl(l)]);
        };
        ld(0, kf[0], qf[0]);
        sched_fence();
#pragma unroll
        for (int t = 0; t < 2; ++t) fac[t] = diag_decay(g, PR[SET][t], lr, lg);
#pragma unroll
        for (int t = 2; t < 5; ++t) fac[t] = offdiag_p(g, PR[SET][t], PJ[SET][t], lr, lg, f4{1.f, 1.f, 1.f, 1.f});
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          if (kk < 3) ld(kk + 1, kf[(kk + 1) & 1], qf[(kk + 1) & 1]);
          if constexpr (L2N) {  // unit keys: columns scale by 1 / |k_j| (rows by 1 / |q_r| at the outputs);
            if (kk == 2) {      // read behind the last fragments so no fragment load waits for them
#pragma unroll
              for (int t = 0; t < 5; ++t) rkc[t] = *reinterpret_cast<const f4*>(&g.rk[16 * PJ[SET][t] + 4 * lg]);
            }
          }
          sched_fence();
#pragma unroll
          for (int t = 0; t < 5; ++t) acc[t] = mfma32(kf[kk & 1][PJ[SET][t]], qf[kk & 1][PR[SET][t]], acc[t]);
          sched_fence();
        }
      }
#pragma unroll
      for (int t = 0; t < 5; ++t) {
        if constexpr (L2N) fac[t] *= rkc[t];
        *reinterpret_cast<h4*>(&sm.p[16 * PR[SET][t] + lr][16 * PJ[SET][t] + 4 * swl4(l)]) = to_h4(fac[t] * acc[t]);
      }
    }
    __syncthreads();
    {
      const int kb2 = kbuf(c + 2), ab = (int)(c & 1);
      const Gates& g = sm.gt[kb2];
      f4 fac[3], acc[3], rkc[3];
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        fac[t] = offdiag_neg_a(g, AR[SET][t], AJ[SET][t], lr, lg, f4{1.f, 1.f, 1.f, 1.f});
        acc[t] = f4{0.f, 0.f, 0.f, 0.f};
      }
      {
        h8 kf[2][4];
        auto ld = [&](int kk, h8 (&k4)[4]) {
#pragma unroll
          for (int J = SET; J < 4; ++J) k4[J] = lds8(&sm.k[kb2][16 * J + lr][32 * kk + 8 * swl(l)]);
        };
        ld(0, kf[0]);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          if (kk < 3) ld(kk + 1, kf[(kk + 1) & 1]);
          if constexpr (L2N) {  // unit keys: rows and columns scale by 1 / |k|, read behind the fragments
            if (kk == 2) {
#pragma unroll
              for (int t = 0; t < 3; ++t)
                rkc[t] = g.rk[16 * AR[SET][t] + lr] * *reinterpret_cast<const f4*>(&g.rk[16 * AJ[SET][t] + 4 * lg]);
            }
          }
          sched_fence();
#pragma unroll
          for (int t = 0; t < 3; ++t) acc[t] = mfma32(kf[kk & 1][AJ[SET][t]], kf[kk & 1][AR[SET][t]], acc[t]);
          sched_fence();
        }
      }
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        if constexpr (L2N) fac[t] *= rkc[t];
        *reinterpret_cast<h4*>(&sm.an[ab][an_idx(AR[SET][t], AJ[SET][t])][lr][4 * lg]) = to_h4(fac[t] * acc[t]);
      }
    }
    __syncthreads();
  }
}

// A ragged batch is processed longest sequence first, so that the short ones fill in behind the
// long ones instead of leaving a tail of long workgroups (workgroups are dispatched in id order,
// round-robin over the XCDs).  Stream slot s (the workgroup id over NT, after the XCD remap) is
// given the stream of dispatch rank r: the slot's position in dispatch order (round-robin over
// the eight XCD groups of slots when the remap applies).  Rank r is value head r % H of the
// sequence ranked r / H by length (descending, lower index first among equals).  Every slot
// gets a distinct stream.  The lengths are ranked in the LDS of the P tile, before it is
// cleared.  Needs B <= NTH; returns b * H + h of the slot's stream.
__device__ __forceinline__ int64_t longest_first(Smem& sm, const ChunkArgs& p, int64_t slot, bool xcd_remap, int tid) {
  const int64_t S = p.B * p.H;
  const int64_t r = xcd_remap ? 8 * (slot % (S / 8)) + slot / (S / 8) : slot;
  const int q = (int)(r / p.H);
  int* len = reinterpret_cast<int*>(&sm.p[0][0]);  // NTH lengths (-1 past B), then the answer
  int* win = len + NTH;
  const int nb = (int)p.B, nb4 = (nb + 3) & ~3;
  if (tid < nb) {
    const int64_t t0 = min(max((int64_t)p.cu_seqlens[tid], (int64_t)0), p.T);
    const int64_t t1 = min(max((int64_t)p.cu_seqlens[tid + 1], t0), p.T);
    len[tid] = (int)(t1 - t0);
  } else if (tid < nb4) {
    len[tid] = -1;  // never longer than, nor equal to, a real length
  }
  __syncthreads();
  if (tid < nb) {
    const int lj = len[tid];
    int rank = 0;
    for (int i = 0; i < nb4; i += 4) {
      const int4 l4 = *reinterpret_cast<const int4*>(&len[i]);
      rank += (l4.x > lj || (l4.x == lj && i < tid)) + (l4.y > lj || (l4.y == lj && i + 1 < tid)) +
              (l4.z > lj || (l4.z == lj && i + 2 < tid)) + (l4.w > lj || (l4.w == lj && i + 3 < tid));
    }
    if (rank == q) *win = tid;
  }
  __syncthreads();
  const int64_t bh = (int64_t)(*win) * p.H + r % p.H;
  __syncthreads();  // every wave has read the answer before the P tile is cleared
  return bh;
}

template <typename TOut, bool RAW, bool L2N>
__global__ __launch_bounds__(NTH, 1) void gdn_chunk_mfma_kernel(ChunkArgs p) {
  __shared__ Smem sm;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63;

  // XCD-aware placement: consecutive workgroup ids are dealt round-robin over the 8 XCDs;
  // remap so the NT slices of a stream get ids that land on the same XCD.
  const unsigned nblk = gridDim.x;
  unsigned bid = blockIdx.x;
  const bool xcd_remap = nblk % (8 * NT) == 0;
  if (xcd_remap) bid = (bid % 8) * (nblk / 8) + bid / 8;
  const int c0 = (int)(bid % NT) * DVT;
  int64_t bh = bid / NT;
  if (p.cu_seqlens && p.B <= NTH) bh = longest_first(sm, p, bh, xcd_remap, tid);
  // value head h of sequence b reads query/key head h / (H / Hqk)
  const int64_t b = bh / p.H, h = bh % p.H, hq = h / (p.H / p.Hqk);
  Stream str;
  str.st = bh;
  if (p.cu_seqlens) {  // offsets clamped into [0, T]: any table keeps every access inside the tensors
    const int64_t t0 = min(max((int64_t)p.cu_seqlens[b], (int64_t)0), p.T);
    const int64_t t1 = min(max((int64_t)p.cu_seqlens[b + 1], t0), p.T);
    str.T = t1 - t0;
    str.qk = (p.Hqk * t0 + hq * str.T) * D;
    str.tok = p.H * t0 + h * str.T;
  } else {
    str.T = p.T;
    str.qk = (b * p.Hqk + hq) * p.T * D;
    str.tok = bh * p.T;
  }
  const int64_t nchunks = (str.T + C - 1) / C;

  // T and P start at zero; their upper blocks are never written
  for (int e = tid; e < 2 * C * LC / 8; e += NTH) reinterpret_cast<v4u*>(&sm.t[0][0][0])[e] = v4u{0u, 0u, 0u, 0u};
  for (int e = tid; e < C * LK / 8; e += NTH) reinterpret_cast<v4u*>(&sm.p[0][0])[e] = v4u{0u, 0u, 0u, 0u};

  // Every role runs nchunks + 2 iterations of two barriers after one initial barrier.  Waves w,
  // w + 4 and w + 8 share a SIMD: each chain (0, 1) shares its SIMD with an output wave (4, 5)
  // and a staging wave (8, 9); the producers (2, 3, 6, 7, 10, 11) fill the other two SIMDs.
  switch (w) {
    case 0:
    case 1:
      __builtin_amdgcn_s_setprio(2);
      chain_role(sm, p, str, c0, w, l, nchunks);
      break;
    case 2: tdiag_role<0, L2N>(sm, l, nchunks); break;
    case 3: tdiag_role<2, L2N>(sm, l, nchunks); break;
    case 4: out_role<TOut, 0, L2N>(sm, p, str, c0, l, nchunks); break;
    case 5: out_role<TOut, 2, L2N>(sm, p, str, c0, l, nchunks); break;
    case 6: key_toff_role<0, L2N>(sm, p, str, l, nchunks); break;
    case 7: key_toff_role<1, L2N>(sm, p, str, l, nchunks); break;
    case 8: gates_qv_role<RAW, L2N>(sm, p, str, c0, l, nchunks); break;
    case 9: q_role<RAW, L2N>(sm, p, str, l, nchunks); break;
    case 10: pa_role<0, L2N>(sm, l, nchunks); break;
    default: pa_role<1, L2N>(sm, l, nchunks); break;
  }
}

}  // namespace

bool chunk_mfma_supported(const ChunkArgs& a) {
  // buffer-descriptor offsets are 32-bit: one stream's q/k/v and o must stay under 2 GiB
  return a.in_dtype == GDN_BF16 && a.D == D && a.chunk == C && a.T * D * 4 < (INT64_C(1) << 31);
}

template <typename TOut>
void launch_variant(const ChunkArgs& a, dim3 grid, dim3 block, hipStream_t s) {
  if (a.raw_gates) {
    if (a.qk_l2norm) hipLaunchKernelGGL((gdn_chunk_mfma_kernel<TOut, true, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((gdn_chunk_mfma_kernel<TOut, true, false>), grid, block, 0, s, a);
  } else {
    if (a.qk_l2norm) hipLaunchKernelGGL((gdn_chunk_mfma_kernel<TOut, false, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((gdn_chunk_mfma_kernel<TOut, false, false>), grid, block, 0, s, a);
  }
}

hipError_t launch_chunk_mfma(const ChunkArgs& a, bool kda, hipStream_t s) {
  if (kda) return launch_kda_mfma(a, s);
  const int64_t blocks = a.B * a.H * NT;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks), block(NTH);
  if (a.out_dtype == GDN_BF16) launch_variant<__hip_bfloat16>(a, grid, block, s);
  else launch_variant<float>(a, grid, block, s);
  return hipGetLastError();
}

}  // namespace gdn
