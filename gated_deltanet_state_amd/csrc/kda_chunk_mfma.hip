// kda_chunk_mfma.hip -- matrix-core chunkwise prefill of KDA (per-channel decay) for gfx950
// (bf16 inputs, d_k = d_v = 128, chunk = 64, fp32 state and accumulation).
//
// KDA replaces the scalar gate of the gated delta rule by one forget rate per key channel,
// S_t = S_{t-1} Diag(alpha_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T ("From Traditional
// Attention to hybrid ones", section 7).  Its chunkwise form ("Hybrid Linear Attention
// Architecture Design Explained", section 4) in the d_v x d_k convention, with the
// per-channel prefix G_r = sum_{s<=r} log alpha_s in R^{d_k} and Gamma_r = e^{G_r}:
//   A = strict_tril(diag(beta) (K*Gamma)(K/Gamma)^T),  X = diag(beta)(V - (K*Gamma) S^T)
//   (I + A) U = X
//   O = (Q*Gamma) S^T + tril((Q*Gamma)(K/Gamma)^T) U
//   S <- S Diag(Gamma_63) + U^T (K * e^{G_63 - G})
// The page notes that the division form needs overflow protection.  Here every factor
// e^{G_r - G_j} (j <= r, always <= 1) is split at a reference point between j and r so that
// both half-precision operands stay bounded:
//   * off the diagonal 16-token blocks (j in block J < R = block of r) the split point is the
//     end of block J: (k_r e^{G_r - G_end(J)}) . (k_j e^{G_end(J) - G_j}), both factors <= 1
//     for any gate strength;
//   * inside a diagonal block the split point is its middle token m, with factors up to
//     e^{G_start - G_m} and e^{G_m - G_end} per channel.  While both stay below e^8 (and the
//     rows times the factors stay in half range) the block runs on the matrix cores like the
//     others.  A block whose gates are stronger is flagged when its chunk is staged: its rows
//     take the block start as their reference instead (all their factors <= 1), and its two
//     diagonal 16x16 tiles of A and P are formed exactly in fp32, each factor
//     e^{G_r - G_j} <= 1 computed for its own pair (r, j) and channel.  So every finite gate
//     <= 0 gives finite, accurate results; strong gates only cost the flagged blocks' extra
//     work.
// Work decomposition as in the scalar-gate kernel (a workgroup per stream and 32 value rows,
// 8 wavefronts), without its cross-chunk pipelining: the per-channel operand tiles fill the
// LDS.  Per chunk: stage (log-gate prefix per channel, scaled operand tiles) | Gram/score
// tiles, diagonal inverses, X, O | substitution | O += P U and the state hand-off.
// Two-kernel form (when the caller passes a workspace): a preparation kernel writes each chunk's
// state-independent operands once per stream as a record, and a sequential kernel streams the
// records through LDS (double-buffered, LDS-direct copies) instead of the four value-slice
// workgroups each staging and multiplying them.
#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>

#include <mutex>

#include "gdn_internal.h"
#include "gdn_mfma_common.h"

namespace gdn {
namespace {

using namespace mfma;

constexpr int D = 128;       // head dimension (d_k = d_v)
constexpr int C = 64;        // chunk length
constexpr int DVT = 32;      // value rows per workgroup
constexpr int NT = D / DVT;  // workgroups per stream
constexpr int NTH = 512;     // threads per workgroup
constexpr int LQ = D + 8;    // row stride (halves) of [token][channel] tiles
constexpr int LC = C + 8;    // row stride (halves) of [channel][token] and [token][token] tiles
constexpr int LT = 24;       // row stride (halves) of 16x16 blocks
constexpr int LG = D + 4;    // row stride (floats) of the fp32 prefix G[token][channel]

// Reference point of the rows of block R: its middle token m(R) = 16 R + 7, or for a flagged
// block (strong gates, see DiagFlags) the state entering it, G_ref = G_{16R-1} (0 for R = 0).
struct alignas(16) Tables {
  alignas(16) float beta[C];
  alignas(16) float em[4][D];     // e^{G_ref(R)}: turns k e^{G - G_ref} into k e^{G}
  alignas(16) float fm[4][4][D];  // fm[R][J] = e^{G_ref(R) - G_end(J)} <= 1, J < R, G_end(J) = G_{16J+15}
  alignas(16) float gc[D];        // e^{G_63}
};

// Blocks whose diagonal tiles are formed exactly (bit R), and the largest |q|, |k| element of
// each block's rows (one entry per staging wavefront: keys 0..3, queries 4..7).
struct alignas(16) DiagFlags {
  float rowmax[8];
  int bits;
};
// A block runs its diagonal tiles on the matrix cores while both middle-token factors stay
// below e^kDiagExp (so the small ones stay normal halves) and rows times factors below
// kDiagLimit (half range with margin).
constexpr float kDiagExp = 8.f;
constexpr float kDiagLimit = 16384.f;

struct alignas(16) Products {
  alignas(16) _Float16 p[C][LC];        // tril((Q*Gamma)(K/Gamma)^T), inclusive
  alignas(16) _Float16 an[C][LC];       // -A, off-diagonal 16x16 blocks
  alignas(16) _Float16 td[4][16][LT];   // inverses of the diagonal blocks of (I + A), row-major
  alignas(16) _Float16 nt[4][16][LT];   // scratch: transposed diagonal blocks of A
  alignas(16) _Float16 u[DVT][LC];      // U [d_v][token]
};

struct alignas(16) Prefix {
  alignas(16) float G[C][LG];           // inclusive prefix of log alpha per channel
  alignas(16) float tot[17][D];         // sums over groups of 4 tokens; then their exclusive prefix and the total
};

struct alignas(16) Smem {
  alignas(16) _Float16 ql[C][LQ];   // q_r e^{G_r - G_m(R)}
  alignas(16) _Float16 kl[C][LQ];   // k_r e^{G_r - G_m(R)}
  alignas(16) _Float16 kd[C][LQ];   // k_j e^{G_m(J) - G_j}         (A operand, diagonal blocks)
  alignas(16) _Float16 kr[C][LQ];   // k_j e^{G_end(J) - G_j} <= |k|  (A operand, off the diagonal)
  alignas(16) _Float16 kt[D][LC];   // k_c e^{G_63 - G_c} <= |k|, transposed [d_k][token], swizzled
  alignas(16) _Float16 s[DVT][LQ];  // fp16 copy of the state slice [d_v][d_k]
  alignas(16) _Float16 v[C][DVT + 8];
  union {                           // the prefix lives only while the chunk is staged
    Prefix pf;
    Products pr;
  };
  Tables tb;
  alignas(16) _Float16 fb[4][2][16][16];  // flagged blocks: exact diagonal tiles of A (x beta) and P
  DiagFlags df;
};

struct Streams {
  __amdgpu_buffer_rsrc_t qk, g, v, beta;
};

__device__ __forceinline__ Streams make_streams(const ChunkArgs& p, int64_t bh, bool is_q) {
  const int64_t tok = bh * p.T;
  const int bytes_qkv = (int)(p.T * D * 2);
  Streams s;
  s.qk = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)(is_q ? p.q : p.k) + tok * D), 0, bytes_qkv, kRsrcWord3);
  s.g = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)p.log_alpha + tok * D), 0, bytes_qkv, kRsrcWord3);
  s.v = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)p.v + tok * D), 0, bytes_qkv, kRsrcWord3);
  s.beta = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)p.beta + tok), 0, (int)(p.T * 2), kRsrcWord3);
  return s;
}

// Threads 0..255 stage keys, log-gates, values and beta; threads 256..511 queries.  Tokens
// past the end of the stream read as zeros (identity steps).
struct Stage {
  v4u x[4];   // q or k: rows 4*(t/16)+i, channels 8*(t%16)..+7
  v4u g[4];   // log alpha, same layout (key threads)
  v4u v;      // key threads: row t/4, value channels c0 + 8*(t%4)..+7
  unsigned short beta;
};

__device__ __forceinline__ void stage_load(Stage& st, const Streams& sr, int64_t t0, int tid, int c0) {
  const int t = tid & 255, g8 = t & 15, rq = t >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int off = (int)(((t0 + 4 * rq + i) * D + 8 * g8) * 2);
    st.x[i] = __builtin_amdgcn_raw_buffer_load_b128(sr.qk, off, 0, 0);
    if (tid < 256) st.g[i] = __builtin_amdgcn_raw_buffer_load_b128(sr.g, off, 0, 0);
  }
  if (tid < 256)
    st.v = __builtin_amdgcn_raw_buffer_load_b128(sr.v, (int)(((t0 + (t >> 2)) * D + c0 + 8 * (t & 3)) * 2), 0, 0);
  if (tid < C) st.beta = __builtin_amdgcn_raw_buffer_load_b16(sr.beta, (int)((t0 + tid) * 2), 0, 0);
}

__device__ __forceinline__ float bf_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf_at(v4u x, int e) { return (e & 1) ? bf_hi(x[e >> 1]) : bf_lo(x[e >> 1]); }

// Half-precision operand fragment (8 channels) scaled per channel by an fp32 table row,
// rounded to nearest once.
__device__ __forceinline__ h8 scale8(h8 a, const float* tab) {
  const f4 t0 = *reinterpret_cast<const f4*>(tab), t1 = *reinterpret_cast<const f4*>(tab + 4);
  h8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[i] = (_Float16)((float)a[i] * t0[i]);
    r[4 + i] = (_Float16)((float)a[4 + i] * t1[i]);
  }
  return r;
}

// Inverse of (I + N), N = A_JJ strictly lower, on 16x16x16 MFMAs (see the scalar-gate kernel).
__device__ __forceinline__ void invert_diag(Smem& sm, int J, f4 rowN, int lr, int lg) {
  const f4 zero = {0.f, 0.f, 0.f, 0.f};
  f4 eye;
#pragma unroll
  for (int i = 0; i < 4; ++i) eye[i] = (4 * lg + i == lr) ? 1.f : 0.f;
  const h4 rN = to_h4(rowN);
#pragma unroll
  for (int i = 0; i < 4; ++i) sm.pr.nt[J][4 * lg + i][lr] = rN[i];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const h4 cN = *reinterpret_cast<const h4*>(&sm.pr.nt[J][lr][4 * lg]);
  const f4 n2c = mfma16(rN, cN, zero), n2r = mfma16(cN, rN, zero);
  const h4 n2ch = to_h4(n2c), n2rh = to_h4(n2r);
  const f4 n4c = mfma16(n2rh, n2ch, zero), n4r = mfma16(n2ch, n2rh, zero);
  const f4 n8c = mfma16(to_h4(n4r), to_h4(n4c), zero);
  const f4 p1r = mfma16(to_h4(n2c + eye), to_h4(eye - rowN), zero);
  const f4 p2r = mfma16(to_h4(n4c + eye), to_h4(p1r), zero);
  const f4 tr = mfma16(to_h4(n8c + eye), to_h4(p2r), zero);
  *reinterpret_cast<h4*>(&sm.pr.td[J][lr][4 * lg]) = to_h4(tr);
}

// Job codes: kind << 4 | R << 2 | J.  kind 0: A tile (R, J); kind 1: P tile (R, J); kind 2:
// output tile O^T (token block R, value block J), whose accumulator is kept for the P U step.
constexpr int job(int kind, int R, int J) { return (kind << 4) | (R << 2) | J; }
constexpr int kNone = -1;

template <int J0, int J1, int J2, int J3, int J4>
struct Jobs {
  static constexpr int at[5] = {J0, J1, J2, J3, J4};
};

// Gram / score tile (M = j, N = r): the lane holds r = 16 R + lr, j = 16 J + 4 lg + i.
template <class L>
__device__ __forceinline__ void produce(Smem& sm, int l, f4* Oacc, int flags) {
  const int lr = l & 15, lg = l >> 4;
  f4 acc[5];
#pragma unroll
  for (int t = 0; t < 5; ++t) acc[t] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int ch = 32 * kk + 8 * lg;  // channels of this lane's fragments
#pragma unroll
    for (int t = 0; t < 5; ++t) {
      const int jb = L::at[t];
      if (jb == kNone) continue;
      const int kind = jb >> 4, R = (jb >> 2) & 3, J = jb & 3;
      if (kind == 2) {  // O^T[dv][c] += sum S[dv][ch] (Q Gamma)[c][ch]: B operand = ql rows c * e^{G_m(R)}
        const h8 qf = frag8(&sm.ql[0][0], LQ, 16 * R, 32 * kk, l);
        const h8 qb = scale8(qf, &sm.tb.em[R][ch]);
        acc[t] = mfma32(frag8(&sm.s[0][0], LQ, 16 * J, 32 * kk, l), qb, acc[t]);
      } else {
        const _Float16* Am = (R == J) ? &sm.kd[0][0] : &sm.kr[0][0];
        const _Float16* Bm = kind ? &sm.ql[0][0] : &sm.kl[0][0];
        h8 b = frag8(Bm, LQ, 16 * R, 32 * kk, l);
        if (R != J) b = scale8(b, &sm.tb.fm[R][J][ch]);
        acc[t] = mfma32(frag8(Am, LQ, 16 * J, 32 * kk, l), b, acc[t]);
      }
    }
  }
#pragma unroll
  for (int t = 0, no = 0; t < 5; ++t) {
    const int jb = L::at[t];
    if (jb == kNone) continue;
    const int kind = jb >> 4, R = (jb >> 2) & 3, J = jb & 3;
    if (kind == 2) {
      Oacc[no++] = acc[t];
      continue;
    }
    const int r = 16 * R + lr, j0 = 16 * J + 4 * lg;
    f4 a = acc[t];
    if (R == J && ((flags >> R) & 1)) {
      // flagged block: the exact tile formed while the chunk was staged (masked, A times beta)
      const h4 x = *reinterpret_cast<const h4*>(&sm.fb[R][kind][lr][4 * lg]);
      a = f4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
    } else {
      if (R == J) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = j0 + i;
          if (kind ? (j > r) : (j >= r)) a[i] = 0.f;
        }
      }
      if (kind == 0) a *= sm.tb.beta[r];
    }
    if (kind == 1) {
      *reinterpret_cast<h4*>(&sm.pr.p[r][j0]) = to_h4(a);
    } else {
      if (R == J)
        invert_diag(sm, J, a, lr, lg);
      else
        *reinterpret_cast<h4*>(&sm.pr.an[r][j0]) = to_h4(-a);
    }
  }
}

// Producer wavefronts 2..7: 20 A / P tiles (with the four diagonal inverses) and the 8 output
// tiles; the O tiles of a wavefront are (R, J) = (token block, value block).
using JobsW2 = Jobs<job(0, 0, 0), job(0, 1, 0), job(0, 2, 0), job(0, 3, 0), job(2, 0, 0)>;
using JobsW3 = Jobs<job(1, 0, 0), job(1, 1, 0), job(1, 2, 0), job(1, 3, 0), job(2, 0, 1)>;
using JobsW4 = Jobs<job(0, 1, 1), job(0, 2, 1), job(0, 3, 1), job(1, 1, 1), job(2, 1, 0)>;
using JobsW5 = Jobs<job(1, 2, 1), job(1, 3, 1), job(0, 2, 2), job(2, 1, 1), job(2, 2, 0)>;
using JobsW6 = Jobs<job(1, 2, 2), job(1, 3, 2), job(0, 3, 3), job(2, 2, 1), job(2, 3, 0)>;
using JobsW7 = Jobs<job(0, 3, 2), job(1, 3, 3), job(2, 3, 1), kNone, kNone>;

// O tiles owned by wavefront w (matching the lists above): count, and (token block, value block).
__device__ __forceinline__ int o_count(int w) { return (w == 5 || w == 6) ? 2 : 1; }
__device__ __forceinline__ void o_tile(int w, int t, int& cb, int& db) {
  // w2: (0,0)  w3: (0,1)  w4: (1,0)  w5: (1,1),(2,0)  w6: (2,1),(3,0)  w7: (3,1)
  const int idx = (w == 2) ? 0 : (w == 3) ? 1 : (w == 4) ? 2 : (w == 5) ? 3 + t : (w == 6) ? 5 + t : 7;
  cb = idx >> 1;
  db = idx & 1;
}

// Blocks flagged as too strongly gated for the middle-token split (bits of `flags`): after the
// regular staging, each thread stages its own rows of those blocks again with the state
// entering the block, G_b = G_{16R-1} (0 for the first block), as the rows' reference, so every
// factor is <= 1: k_r e^{G_r - G_b}, k_r e^{G_end - G_r}, k_r e^{G_63 - G_r}, q_r e^{G_r - G_b},
// and the tables e^{G_b}, e^{G_b - G_end(J)}.  The middle-token keys of those blocks are unused
// (zeroed): their diagonal 16x16 tiles of A and P are formed exactly instead,
// A_rj = beta_r sum_c k_rc k_jc e^{G_rc - G_jc} (j < r), P_rj = sum_c q_rc k_jc e^{G_rc - G_jc}
// (j <= r), each factor (<= 1) computed in fp32 from the prefix of its own pair and channel.
// Rows are read again from the inputs (zeros past the end of the stream).  A call outside the
// regular path, so the registers of that path are not shaped by it; every thread calls it.
struct FlagArgs {  // what the slow path reads besides the LDS (passed by value: no copy of the kernel arguments)
  const void *q, *k, *beta;
  int64_t T, bh, t0;
};
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* base, const FlagArgs& f, int64_t per_tok) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)base + f.bh * f.T * per_tok), 0,
                                           (int)(f.T * per_tok * 2), kRsrcWord3);
}
__device__ __noinline__ void restage_flagged(Smem& sm, FlagArgs f, int flags, int tid) {
  const int t = tid & 255, g8 = t & 15, rq = t >> 4, R = rq >> 2;
  const int64_t t0 = f.t0;
  const auto rows = row_rsrc(tid >= 256 ? f.q : f.k, f, D);
  if ((flags >> R) & 1) {
    const float* Ge = &sm.pf.G[16 * R + 15][8 * g8];
    const float* Gl = &sm.pf.G[C - 1][8 * g8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * rq + i;
      const v4u x = __builtin_amdgcn_raw_buffer_load_b128(rows, (int)(((t0 + row) * D + 8 * g8) * 2), 0, 0);
      const float* Gr = &sm.pf.G[row][8 * g8];
      h8 a, b, c, d;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = bf_at(x, e), gb = R ? sm.pf.G[16 * R - 1][8 * g8 + e] : 0.f;
        const float er = __expf(fminf(Ge[e] - Gr[e], 0.f));                 // e^{G_end - G_r}
        a[e] = (_Float16)(v * __expf(fminf(Gr[e] - gb, 0.f)));              // e^{G_r - G_b}
        b[e] = (_Float16)(v * er);
        c[e] = (_Float16)(v * er * __expf(fminf(Gl[e] - Ge[e], 0.f)));      // e^{G_63 - G_r}
        d[e] = (_Float16)0.f;
      }
      if (tid < 256) {
        *reinterpret_cast<h8*>(&sm.kl[row][8 * g8]) = a;
        *reinterpret_cast<h8*>(&sm.kd[row][8 * g8]) = d;
        *reinterpret_cast<h8*>(&sm.kr[row][8 * g8]) = b;
#pragma unroll
        for (int e = 0; e < 8; ++e) sm.kt[8 * g8 + e][kt_col(8 * g8 + e, row)] = c[e];
      } else {
        *reinterpret_cast<h8*>(&sm.ql[row][8 * g8]) = a;
      }
    }
  }
  if (tid >= 384) {  // tables of the flagged blocks, one channel per thread (the regular writers)
    const int ch = tid - 384;
    for (int R2 = 0; R2 < 4; ++R2) {
      if (!((flags >> R2) & 1)) continue;
      const float gb = R2 ? sm.pf.G[16 * R2 - 1][ch] : 0.f;
      sm.tb.em[R2][ch] = __expf(gb);
      for (int J2 = 0; J2 < R2; ++J2) sm.tb.fm[R2][J2][ch] = __expf(fminf(gb - sm.pf.G[16 * J2 + 15][ch], 0.f));
    }
  }
  // exact diagonal tiles: two threads per pair (r, j), 64 channels each
  const int pr = tid >> 1, r = pr >> 4, j = pr & 15, c0 = 64 * (tid & 1);
  const auto krs = row_rsrc(f.k, f, D), qrs = row_rsrc(f.q, f, D), brs = row_rsrc(f.beta, f, 1);
  for (int B = 0; B < 4; ++B) {
    if (!((flags >> B) & 1)) continue;
    const int64_t tr = t0 + 16 * B + r, tj = t0 + 16 * B + j;
    float sa = 0.f, sp = 0.f;
    if (j <= r) {
      for (int c = c0; c < c0 + 64; c += 8) {
        const v4u kr = __builtin_amdgcn_raw_buffer_load_b128(krs, (int)((tr * D + c) * 2), 0, 0);
        const v4u qr = __builtin_amdgcn_raw_buffer_load_b128(qrs, (int)((tr * D + c) * 2), 0, 0);
        const v4u kj = __builtin_amdgcn_raw_buffer_load_b128(krs, (int)((tj * D + c) * 2), 0, 0);
        const float* gr = &sm.pf.G[16 * B + r][c];
        const float* gj = &sm.pf.G[16 * B + j][c];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float w = bf_at(kj, e) * __expf(fminf(gr[e] - gj[e], 0.f));
          sa = fmaf(bf_at(kr, e), w, sa);
          sp = fmaf(bf_at(qr, e), w, sp);
        }
      }
    }
    sa += __shfl_xor(sa, 1, 64);
    sp += __shfl_xor(sp, 1, 64);
    if ((tid & 1) == 0) {
      const float beta = bf_lo(__builtin_amdgcn_raw_buffer_load_b16(brs, (int)(tr * 2), 0, 0));
      sm.fb[B][0][r][j] = (_Float16)(r > j ? beta * sa : 0.f);
      sm.fb[B][1][r][j] = (_Float16)sp;
    }
  }
}

// Stages one chunk (ends with a barrier): the per-channel prefix of log alpha (stage 1, 2a,
// 2b), then the scaled operand tiles, the per-channel tables, the value slice and beta
// (stage 3) from the registers of stage_load.  Every thread of the workgroup calls it.
__device__ __forceinline__ int stage_chunk(Smem& sm, const Stage& st, const ChunkArgs& p, int64_t bh, int64_t t0,
                                           int tid, int w, int l) {
  const int t = tid & 255, g8 = t & 15, rq = t >> 4;
  // ---- stage 1: per-channel prefix of log alpha over each group of 4 tokens; the largest row
  // element of each wavefront's block (keys: waves 0..3, queries: waves 4..7, block w % 4)
  float gl[4][8];
  {
    // bf16 magnitudes order like their bit patterns: an integer max, two per dword, then a DPP
    // max over the wavefront (lane 63 ends with it)
    typedef unsigned short us2 __attribute__((ext_vector_type(2)));
    us2 m2 = {0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int d = 0; d < 4; ++d) m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(us2, st.x[i][d] & 0x7fff7fffu));
    int mx = m2[0] > m2[1] ? m2[0] : m2[1];
#define GDN_DPP_MAX(ctrl, rows) mx = max(mx, __builtin_amdgcn_update_dpp(mx, mx, ctrl, rows, 0xf, false))
    GDN_DPP_MAX(0x111, 0xf);  // row_shr:1
    GDN_DPP_MAX(0x112, 0xf);  // row_shr:2
    GDN_DPP_MAX(0x114, 0xf);  // row_shr:4
    GDN_DPP_MAX(0x118, 0xf);  // row_shr:8
    GDN_DPP_MAX(0x142, 0xa);  // row_bcast:15
    GDN_DPP_MAX(0x143, 0xc);  // row_bcast:31
#undef GDN_DPP_MAX
    const int wmax = __builtin_amdgcn_readlane(mx, 63);
    if (l == 0) sm.df.rowmax[w] = __uint_as_float((uint32_t)wmax << 16);
  }
  if (tid < 256) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float a = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a += bf_at(st.g[i], e);
        gl[i][e] = a;
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
      *reinterpret_cast<f4*>(&sm.pf.tot[rq][8 * g8 + 4 * h]) = f4{gl[3][4 * h], gl[3][4 * h + 1], gl[3][4 * h + 2], gl[3][4 * h + 3]};
  }
  __syncthreads();

  // ---- stage 2a: exclusive prefix of the 16 group sums, two channels per lane of wave 4, and
  // their total
  if (w == 4) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    f2 x[16], run = {0.f, 0.f};
#pragma unroll
    for (int qg = 0; qg < 16; ++qg) x[qg] = *reinterpret_cast<const f2*>(&sm.pf.tot[qg][2 * l]);
#pragma unroll
    for (int qg = 0; qg < 16; ++qg) {
      *reinterpret_cast<f2*>(&sm.pf.tot[qg][2 * l]) = run;
      run += x[qg];
    }
    *reinterpret_cast<f2*>(&sm.pf.tot[16][2 * l]) = run;
  }
  __syncthreads();

  // ---- stage 2b: add the sums of the earlier groups; publish G.  Wave 5 meanwhile flags the
  // blocks too strongly gated for their middle token (G_start - G_m = P_{4R} - P_{4R+2},
  // G_m - G_end = P_{4R+2} - P_{4R+4} for the exclusive group prefix P) or with rows too large
  // for its factors.
  if (w == 5) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    int bits = 0;
#pragma unroll
    for (int R = 0; R < 4; ++R) {
      const f2 p0 = *reinterpret_cast<const f2*>(&sm.pf.tot[4 * R][2 * l]);
      const f2 p2 = *reinterpret_cast<const f2*>(&sm.pf.tot[4 * R + 2][2 * l]);
      const f2 p4 = *reinterpret_cast<const f2*>(&sm.pf.tot[4 * R + 4][2 * l]);
      const f2 e1 = p0 - p2, e2 = p2 - p4;
      const float m = fmaxf(fmaxf(e1[0], e1[1]), fmaxf(e2[0], e2[1]));
      const float rm = fmaxf(sm.df.rowmax[R], sm.df.rowmax[R + 4]);
      const float lim = fminf(kDiagExp, __logf(kDiagLimit / rm));  // rm = 0: +inf, no limit
      if (__ballot(!(m <= lim))) bits |= 1 << R;                 // NaN limit (rm = inf/NaN) flags too
    }
    if (l == 0) sm.df.bits = bits;
  }
  if (tid < 256) {
    const f4 o0 = *reinterpret_cast<const f4*>(&sm.pf.tot[rq][8 * g8]);
    const f4 o1 = *reinterpret_cast<const f4*>(&sm.pf.tot[rq][8 * g8 + 4]);
    const float off[8] = {o0[0], o0[1], o0[2], o0[3], o1[0], o1[1], o1[2], o1[3]};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int e = 0; e < 8; ++e) gl[i][e] += off[e];
#pragma unroll
      for (int h = 0; h < 2; ++h)
        *reinterpret_cast<f4*>(&sm.pf.G[4 * rq + i][8 * g8 + 4 * h]) =
            f4{gl[i][4 * h], gl[i][4 * h + 1], gl[i][4 * h + 2], gl[i][4 * h + 3]};
    }
  }
  __syncthreads();

  // ---- stage 3: scaled operand tiles, tables, values, beta
  const int flags = __builtin_amdgcn_readfirstlane(sm.df.bits);
  {
    const int R = rq >> 2;  // block of this thread's 4 tokens
    const float* Gm = &sm.pf.G[16 * R + 7][8 * g8];
    if (tid < 256) {
      const float* Ge = &sm.pf.G[16 * R + 15][8 * g8];
      const float* Gl = &sm.pf.G[C - 1][8 * g8];
      // per channel: e^{G_end - G_m} and e^{G_63 - G_end} (both <= 1); per element one
      // exponential and one reciprocal: e^{G_end - G_r} = e^{G_end - G_m} / e^{G_r - G_m}
      float cem[8], c63[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        cem[e] = __expf(fminf(Ge[e] - Gm[e], 0.f));
        c63[e] = __expf(fminf(Gl[e] - Ge[e], 0.f));
      }
      h8 klh[4], kdh[4], krh[4], kth[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float k = bf_at(st.x[i], e);
          const float el = __expf(gl[i][e] - Gm[e]);          // e^{G_r - G_m}
          const float ie = __builtin_amdgcn_rcpf(el);          // e^{G_m - G_r}
          const float er = fminf(cem[e] * ie, 1.f);            // e^{G_end - G_r} <= 1
          klh[i][e] = (_Float16)(k * el);
          kdh[i][e] = (_Float16)(k * ie);
          krh[i][e] = (_Float16)(k * er);
          kth[i][e] = (_Float16)(k * er * c63[e]);              // e^{G_63 - G_r}
        }
        const int row = 4 * rq + i;
        *reinterpret_cast<h8*>(&sm.kl[row][8 * g8]) = klh[i];
        *reinterpret_cast<h8*>(&sm.kd[row][8 * g8]) = kdh[i];
        *reinterpret_cast<h8*>(&sm.kr[row][8 * g8]) = krh[i];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        h4 col;
        col[0] = kth[0][e]; col[1] = kth[1][e]; col[2] = kth[2][e]; col[3] = kth[3][e];
        *reinterpret_cast<h4*>(&sm.kt[8 * g8 + e][kt_col(8 * g8 + e, 4 * rq)]) = col;
      }
      *reinterpret_cast<h8*>(&sm.v[t >> 2][8 * (t & 3)]) = bf8_to_h8(st.v);
      if (tid < C) sm.tb.beta[tid] = __uint_as_float(static_cast<uint32_t>(st.beta) << 16);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float* Gr = &sm.pf.G[4 * rq + i][8 * g8];
        h8 qh;
#pragma unroll
        for (int e = 0; e < 8; ++e) qh[e] = (_Float16)(bf_at(st.x[i], e) * __expf(Gr[e] - Gm[e]));
        *reinterpret_cast<h8*>(&sm.ql[4 * rq + i][8 * g8]) = qh;
      }
      if (tid >= 384) {  // tables, one channel per thread
        const int ch = tid - 384;
#pragma unroll
        for (int R2 = 0; R2 < 4; ++R2) {
          const float gm = sm.pf.G[16 * R2 + 7][ch];
          sm.tb.em[R2][ch] = __expf(gm);
#pragma unroll
          for (int J2 = 0; J2 < R2; ++J2) sm.tb.fm[R2][J2][ch] = __expf(fminf(gm - sm.pf.G[16 * J2 + 15][ch], 0.f));
        }
        sm.tb.gc[ch] = __expf(sm.pf.G[C - 1][ch]);
      }
    }
    // blocks too strongly gated for their middle token are staged again, by the same threads
    if (flags) restage_flagged(sm, FlagArgs{p.q, p.k, p.beta, p.T, bh, t0}, flags, tid);
  }
  __syncthreads();
  return flags;
}

// ------------------------------------------------------------------------------------------
// Two-kernel form (used when the caller provides the workspace).  Everything a chunk needs
// that does not depend on the state -- the staged operand tiles, P, -A and the inverses of
// the diagonal blocks of (I + A), the per-channel tables -- is computed once per (stream,
// chunk) by kda_prep_kernel, fully in parallel, into one record of the workspace.  The
// sequential kernel then only stages a record per chunk (plain copies, one chunk ahead) and
// runs X, the substitution, the outputs and the state hand-off.  The single kernel recomputes
// that state-independent work in each of the NT workgroups of a stream, one chunk after
// another.  Both forms run the same arithmetic on the same operands.
// The record is the LDS image the sequential kernel computes from.  Its fp16 tiles store the
// 16-byte chunk c of row r at chunk c ^ swz128(r) (128-wide rows) or c ^ swz64(r) (64-wide
// rows).  A fragment read (lanes on 16 consecutive rows, two adjacent chunks per 32 lanes) and a
// row-major 16-byte copy (two rows of all chunks per 32 lanes) then touch every LDS bank once.
__device__ __forceinline__ int swz128(int r) { return ((r >> 1) & 7) << 1; }
__device__ __forceinline__ int swz64(int r) { return ((r >> 2) & 3) << 1; }
template <int W>
__device__ __forceinline__ int swz(int r) {
  static_assert(W == D || W == C, "tile width");
  return W == D ? swz128(r) : swz64(r);
}
// Element (r, col) of a swizzled W-wide tile.
template <int W, typename T>
__device__ __forceinline__ T* sat(T* base, int r, int col) {
  return base + r * W + 8 * ((col >> 3) ^ swz<W>(r)) + (col & 7);
}
// Operand fragment of a swizzled W-wide tile: rows m0 + l%16, columns k0 + 8 (l/16) .. +7.
template <int W>
__device__ __forceinline__ h8 sfrag8(const _Float16* base, int m0, int k0, int lane) {
  return *reinterpret_cast<const h8*>(sat<W>(base, m0 + (lane & 15), k0 + 8 * (lane >> 4)));
}

struct alignas(16) KdaRec {
  _Float16 kl[C][D];       // k_r e^{G_r - G_m(R)} e^{G_m(R)}, rounded as the single kernel rounds it at use
  _Float16 ql[C][D];       // q_r e^{G_r - G_m(R)} e^{G_m(R)}, likewise
  _Float16 kt[D][C];       // k_c e^{G_63 - G_c}, [d_k][token]
  _Float16 p[C][C];        // tril((Q*Gamma)(K/Gamma)^T), zero above the diagonal blocks
  _Float16 an[6][16][16];  // -A, blocks (R, J), R > J, at R (R - 1) / 2 + J
  _Float16 td[4][16][16];  // inverses of the diagonal blocks of (I + A), row-major
  float gc[D];             // e^{G_63}
  float beta[C];
  uint8_t pad[256];        // whole KiB: the copy into LDS moves 1 KiB per wavefront instruction
};
constexpr int64_t kRecBytes = 65536;  // record stride in the workspace
constexpr int kRecKiB = (int)(sizeof(KdaRec) / 1024);
static_assert(sizeof(KdaRec) == 62 * 1024 && sizeof(KdaRec) <= kRecBytes, "workspace record");

// R and J of block b of the -A record (b = R (R - 1) / 2 + J)
__device__ __forceinline__ void an_block(int b, int& R, int& J) {
  R = b < 1 ? 1 : (b < 3 ? 2 : 3);
  J = b - R * (R - 1) / 2;
}

// A and P tiles (with the four diagonal inverses) of one chunk over the 8 wavefronts.
using PrepW0 = Jobs<job(0, 0, 0), job(0, 1, 0), job(0, 2, 0), kNone, kNone>;
using PrepW1 = Jobs<job(0, 1, 1), job(0, 2, 1), job(0, 3, 0), kNone, kNone>;
using PrepW2 = Jobs<job(0, 2, 2), job(0, 3, 1), job(1, 0, 0), kNone, kNone>;
using PrepW3 = Jobs<job(0, 3, 3), job(0, 3, 2), job(1, 1, 0), kNone, kNone>;
using PrepW4 = Jobs<job(1, 1, 1), job(1, 2, 0), job(1, 2, 1), kNone, kNone>;
using PrepW5 = Jobs<job(1, 2, 2), job(1, 3, 0), kNone, kNone, kNone>;
using PrepW6 = Jobs<job(1, 3, 1), job(1, 3, 2), kNone, kNone, kNone>;
using PrepW7 = Jobs<job(1, 3, 3), kNone, kNone, kNone, kNone>;

static_assert(offsetof(Prefix, tot) >= offsetof(Products, nt), "group sums overlap the record tiles");

// A slab of the two-kernel form: streams bh0 .. bh0 + nbh - 1, chunks c0 .. c0 + nc - 1 of each.
// Its records sit in the workspace at ((bh - bh0) nc + (ci - c0)) * kRecBytes.  The chain kernel
// starts each stream from s_in and leaves the state in s_out (both [nbh, D, D] fp32 from stream
// bh0; s_in null = zeros, s_out null = not kept), so a long sequence runs as consecutive slabs
// with the state carried between them.
struct Slab {
  int64_t bh0, nbh, c0, nc;
  const float* s_in;
  float* s_out;
};

// Records are spread over a grid of at most one workgroup per CU (the LDS holds one); each
// workgroup walks its records in order, staging each one as the single kernel does, forming the
// A and P tiles and writing the record.  The inputs of the next record are loaded while the
// current one is computed (two register sets), and the record writes are never waited for, so
// neither latency reaches the workgroup's critical path.
__device__ __forceinline__ void prep_record(Smem& sm, const Stage& st, const ChunkArgs& p, const Slab& sl, uint8_t* ws,
                                            int64_t rec, int tid, int w, int l) {
  const int flags = stage_chunk(sm, st, p, sl.bh0 + rec / sl.nc, (sl.c0 + rec % sl.nc) * C, tid, w, l);
  l = opaque(l);
  f4 unused[2];
  switch (w) {
    case 0: produce<PrepW0>(sm, l, unused, flags); break;
    case 1: produce<PrepW1>(sm, l, unused, flags); break;
    case 2: produce<PrepW2>(sm, l, unused, flags); break;
    case 3: produce<PrepW3>(sm, l, unused, flags); break;
    case 4: produce<PrepW4>(sm, l, unused, flags); break;
    case 5: produce<PrepW5>(sm, l, unused, flags); break;
    case 6: produce<PrepW6>(sm, l, unused, flags); break;
    default: produce<PrepW7>(sm, l, unused, flags); break;
  }
  __syncthreads();
  KdaRec* out = reinterpret_cast<KdaRec*>(ws + rec * kRecBytes);
  for (int e = tid; e < C * D / 8; e += NTH) {  // the X and output operands carry e^{G_ref(R)} already
    const int r = e >> 4, cc = 8 * (e & 15);
    const float* em = &sm.tb.em[r >> 4][cc];
    *reinterpret_cast<h8*>(sat<D>(&out->kl[0][0], r, cc)) = scale8(*reinterpret_cast<const h8*>(&sm.kl[r][cc]), em);
    *reinterpret_cast<h8*>(sat<D>(&out->ql[0][0], r, cc)) = scale8(*reinterpret_cast<const h8*>(&sm.ql[r][cc]), em);
  }
  for (int e = tid; e < D * C / 8; e += NTH) {
    const int dk = e >> 3, pc = e & 7;
    *reinterpret_cast<v4u*>(sat<C>(&out->kt[0][0], dk, 8 * pc)) = *reinterpret_cast<const v4u*>(&sm.kt[dk][kt_col(dk, 8 * pc)]);
  }
  for (int e = tid; e < C * C / 8; e += NTH) {
    const int r = e >> 3, pc = e & 7;  // columns 8 pc.. lie in block pc / 2
    v4u x = {0u, 0u, 0u, 0u};
    if ((pc >> 1) <= (r >> 4)) x = *reinterpret_cast<const v4u*>(&sm.pr.p[r][8 * pc]);
    *reinterpret_cast<v4u*>(sat<C>(&out->p[0][0], r, 8 * pc)) = x;
  }
  for (int e = tid; e < 6 * 16 * 2; e += NTH) {
    const int b = e >> 5, rr = (e >> 1) & 15, hh = e & 1;
    int R, J;
    an_block(b, R, J);
    *reinterpret_cast<v4u*>(&out->an[b][rr][8 * hh]) = *reinterpret_cast<const v4u*>(&sm.pr.an[16 * R + rr][16 * J + 8 * hh]);
  }
  for (int e = tid; e < 4 * 16 * 2; e += NTH) {
    const int b = e >> 5, rr = (e >> 1) & 15, hh = e & 1;
    *reinterpret_cast<v4u*>(&out->td[b][rr][8 * hh]) = *reinterpret_cast<const v4u*>(&sm.pr.td[b][rr][8 * hh]);
  }
  if (tid < D) out->gc[tid] = sm.tb.gc[tid];
  if (tid < C) out->beta[tid] = sm.tb.beta[tid];
  // before its first barrier the next record's staging writes only the group sums, which share
  // no bytes with the tiles read above, and the row maxima of its flags; everything else it
  // writes comes after that barrier
}

__global__ __launch_bounds__(NTH, 1) void kda_prep_kernel(ChunkArgs p, uint8_t* ws, Slab sl) {
  __shared__ Smem sm;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63;
  const int64_t nrec = sl.nbh * sl.nc, step = gridDim.x;
  auto load = [&](int64_t rec, Stage& st) {
    if (rec >= nrec) return;
    const int64_t bh = sl.bh0 + rec / sl.nc, ci = sl.c0 + rec % sl.nc;
    stage_load(st, make_streams(p, bh, tid >= 256), ci * C, tid, 0);
  };
  Stage sa, sb;
  int64_t rec = blockIdx.x;
  load(rec, sa);
  load(rec + step, sb);
  for (; rec < nrec; rec += 2 * step) {  // the bounds are uniform over the workgroup
    prep_record(sm, sa, p, sl, ws, rec, tid, w, l);
    load(rec + 2 * step, sa);
    if (rec + step >= nrec) break;
    prep_record(sm, sb, p, sl, ws, rec + step, tid, w, l);
    load(rec + 3 * step, sb);
  }
}

// Output tiles only (the A and P tiles come from the record), same owners as in the single
// kernel.
template <typename TOut>
__global__ __launch_bounds__(NTH, 1) void kda_chunk_mfma_kernel(ChunkArgs p) {
  __shared__ Smem sm;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  int l = tid & 63;

  const unsigned nblk = gridDim.x;
  unsigned bid = blockIdx.x;
  if (nblk % (8 * NT) == 0) bid = (bid % 8) * (nblk / 8) + bid / 8;
  const int tile = bid % NT;
  const int64_t bh = bid / NT;
  const int c0 = tile * DVT;
  const int64_t T = p.T;
  const int64_t nchunks = (T + C - 1) / C;

  f4 S[2];  // wavefront w: S^T tiles (d_k block w, d_v block db)
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
  if (nchunks > 0) stage_load(st, sr, 0, tid, c0);

  TOut* O = static_cast<TOut*>(p.o);
  for (int64_t ci = 0; ci < nchunks; ++ci) {
    const int64_t t0 = ci * C;
    const int n = (int)(T - t0 < C ? T - t0 : C);
    __syncthreads();  // the previous chunk is done with every buffer

    const int flags = stage_chunk(sm, st, p, bh, t0, tid, w, l);
    if (ci + 1 < nchunks) stage_load(st, sr, t0 + C, tid, c0);

    // ---- phase 1: X (waves 0,1), A / P / inverses / O (waves 2..7)
    l = opaque(l);
    int lr = l & 15, lg = l >> 4;
    if (w == 7) {  // zero the upper P blocks that the O += P U step reads: (0,1) and (2,3)
      for (int e = l; e < 2 * 16 * 16; e += 64) {
        const int blk = e >> 8, rr = (e >> 4) & 15, cc = e & 15;
        sm.pr.p[32 * blk + rr][32 * blk + 16 + cc] = (_Float16)0.f;
      }
    }
    f4 X[4], Oacc[2];
    if (w < 2) {
      const int db = w, dv = 16 * db + lr;
#pragma unroll
      for (int i = 0; i < 4; ++i) X[i] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const h8 sb = frag8(&sm.s[0][0], LQ, 16 * db, 32 * kk, l);
        const int ch = 32 * kk + 8 * lg;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          X[i] = mfma32(scale8(frag8(&sm.kl[0][0], LQ, 16 * i, 32 * kk, l), &sm.tb.em[i][ch]), sb, X[i]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = 16 * i + 4 * lg;
        const f4 be = *reinterpret_cast<const f4*>(&sm.tb.beta[c]);
#pragma unroll
        for (int e = 0; e < 4; ++e) X[i][e] = be[e] * ((float)sm.v[c + e][dv] - X[i][e]);
      }
    } else {
      switch (w) {
        case 2: produce<JobsW2>(sm, l, Oacc, flags); break;
        case 3: produce<JobsW3>(sm, l, Oacc, flags); break;
        case 4: produce<JobsW4>(sm, l, Oacc, flags); break;
        case 5: produce<JobsW5>(sm, l, Oacc, flags); break;
        case 6: produce<JobsW6>(sm, l, Oacc, flags); break;
        default: produce<JobsW7>(sm, l, Oacc, flags); break;
      }
    }
    __syncthreads();

    // ---- phase 2: block forward substitution (waves 0,1)
    l = opaque(l);
    lr = l & 15, lg = l >> 4;
    if (w < 2) {
      const int dv = 16 * w + lr;
      h4 an[6], tdf[4];
#pragma unroll
      for (int i = 0, m = 0; i < 4; ++i) {
        tdf[i] = frag4(&sm.pr.td[i][0][0], LT, 0, 0, l);
#pragma unroll
        for (int j = 0; j < i; ++j, ++m) an[m] = frag4(&sm.pr.an[0][0], LC, 16 * i, 16 * j, l);
      }
      h4 Uh[4];
#pragma unroll
      for (int i = 0, m = 0; i < 4; ++i) {
        f4 acc = X[i];
#pragma unroll
        for (int j = 0; j < i; ++j, ++m) acc = mfma16(an[m], Uh[j], acc);
        Uh[i] = to_h4(mfma16(tdf[i], to_h4(acc), f4{0.f, 0.f, 0.f, 0.f}));
        *reinterpret_cast<h4*>(&sm.pr.u[dv][16 * i + 4 * lg]) = Uh[i];
      }
    }
    __syncthreads();

    // ---- phase 3: O += U^T P^T, output (waves 2..7); S <- S Diag(Gamma_63) + U^T (K e^{G_63 - G})
    l = opaque(l);
    lr = l & 15, lg = l >> 4;
    if (w >= 2) {
      const int no = o_count(w);
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        if (t2 >= no) continue;
        int cb, db;
        o_tile(w, t2, cb, db);
        f4 acc = Oacc[t2];
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
          if (kc == 1 && cb < 2) continue;
          acc = mfma32(frag8(&sm.pr.u[0][0], LC, 16 * db, 32 * kc, l), frag8(&sm.pr.p[0][0], LC, 16 * cb, 32 * kc, l), acc);
        }
        const int c = 16 * cb + lr;
        if (c < n) store_o4<TOut>(O, (bh * T + t0 + c) * D + c0 + 16 * db + 4 * lg, acc);
      }
    }
    {
      const bool snap = p.s_ckpt && n == C && ((t0 + n) % p.ckpt_every) == 0;
      const int dkr = 16 * w + lr;
      const int dk = 16 * w + 4 * lg;
      const f4 gcv = *reinterpret_cast<const f4*>(&sm.tb.gc[dk]);
      h8 ka[2];
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) ka[kc] = *reinterpret_cast<const h8*>(&sm.kt[dkr][kt_col(dkr, 32 * kc + 8 * lg)]);
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        f4 acc = S[db] * gcv;
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) acc = mfma32(ka[kc], frag8(&sm.pr.u[0][0], LC, 16 * db, 32 * kc, l), acc);
        S[db] = acc;
        const int dv = 16 * db + lr;
        *reinterpret_cast<h4*>(&sm.s[dv][dk]) = to_h4(acc);
        if (snap) {
          const int64_t idx = (t0 + n) / p.ckpt_every - 1;
          *reinterpret_cast<f4*>(p.s_ckpt + ((bh * p.n_ckpt + idx) * D + c0 + dv) * D + dk) = acc;
        }
      }
    }
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

// ------------------------------------------------------------------------------------------
// Sequential kernel of the two-kernel form.  Per chunk it needs the state-independent operands
// of the chunk's record and its own state slice: X, the substitution, the outputs and the state
// hand-off, on the operands the single kernel uses, in the same order (same bits).  The record
// of chunk c + 1 is copied into the other LDS buffer by LDS-direct loads, issued right after the
// barrier that opens chunk c, so the copy (bound by the LDS write rate) runs under chunk c's
// work instead of before it.  The two buffers are separate LDS objects, which tells the
// compiler that reads of one never wait for the copy into the other.
struct alignas(16) ChainLocal {
  alignas(16) _Float16 s[DVT][D];           // fp16 copy of the state slice [d_v][d_k], swizzled (128-wide)
  alignas(16) _Float16 v[2][C][DVT + 8];    // value slice [token][d_v], by chunk parity
  alignas(16) _Float16 u[DVT][C];           // U [d_v][token], swizzled (64-wide)
  alignas(16) f4 x[4][2][64];               // X tiles (token block, value block), lane-major
};
static_assert(2 * sizeof(KdaRec) + sizeof(ChainLocal) <= 160 * 1024, "LDS budget");

// Barrier between phases of a chunk: the data handed over is written by LDS instructions, so
// each wave waits for its own LDS operations only.  (A barrier with a workgroup release fence
// would also wait for the LDS-direct copy of the next record, which has until the next chunk.)
__device__ __forceinline__ void phase_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Copy of KiB blocks k0, k0 + step, .. below k1 of a record into LDS, one wavefront instruction
// per block (lane l moves bytes 16 l .. 16 l + 15).  A wave issuing these stalls until the
// copy path has taken them (about 50 bytes per cycle per CU), so the copy is issued by waves
// that have nothing else to do at that point.
__device__ __forceinline__ void fetch_blocks(KdaRec& dst, const uint8_t* src, int k0, int k1, int step, int l) {
  uint8_t* d = reinterpret_cast<uint8_t*>(&dst);
  for (int k = k0; k < k1; k += step)
    __builtin_amdgcn_global_load_lds(src + 1024 * k + 16 * l, (__attribute__((address_space(3))) void*)(d + 1024 * k),
                                     16, 0, 0);
}
// Split of the next record's copy: waves 2..7 take blocks below kSplit during the substitution
// (which runs on waves 0 and 1 alone); waves 0 and 1 take the rest at the end of the chunk,
// where they finish earlier than the output waves.
constexpr int kSplit = kRecKiB;
static_assert(kSplit <= kRecKiB, "copy split");

// One chunk: record rc (already in LDS), values in loc.v[vb].  Issues the copy of the next
// record into nx.
template <typename TOut>
__device__ __forceinline__ void chain_chunk(const KdaRec& rc, KdaRec& nx, ChainLocal& loc, int vb, const ChunkArgs& p,
                                            const Streams& sr, const uint8_t* recs, int64_t ci, int64_t cfirst, int64_t cend,
                                            int64_t bh, int c0, int tid, int w, int l, f4 (&S)[2], v4u& vv) {
  const int64_t T = p.T, t0 = ci * C;
  const int n = (int)(T - t0 < C ? T - t0 : C);
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0), lgkmcnt(0): this wave's part of the record has landed
  __syncthreads();  // all parts have; chunk ci - 1 is done with the other buffer and value slot
  const bool more = ci + 1 < cend;  // the slab's records run from chunk cfirst to cend - 1
  const uint8_t* next = recs + (ci + 1 - cfirst) * kRecBytes;
  if (more && tid < 256)
    vv = __builtin_amdgcn_raw_buffer_load_b128(sr.v, (int)((((ci + 1) * C + (tid >> 2)) * D + c0 + 8 * (tid & 3)) * 2), 0, 0);

  // ---- phase 1: one X tile and one O^T = S (Q Gamma)^T tile per wave: token block i = w / 2,
  // value block db = w % 2 (one read of the state fragment serves both)
  l = opaque(l);
  int lr = l & 15, lg = l >> 4;
  f4 oa;
  {
    const int i = w >> 1, db = w & 1, dv = 16 * db + lr;
    f4 x = {0.f, 0.f, 0.f, 0.f};
    oa = x;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const h8 sb = sfrag8<D>(&loc.s[0][0], 16 * db, 32 * kk, l);
      x = mfma32(sfrag8<D>(&rc.kl[0][0], 16 * i, 32 * kk, l), sb, x);
      oa = mfma32(sb, sfrag8<D>(&rc.ql[0][0], 16 * i, 32 * kk, l), oa);
    }
    const int c = 16 * i + 4 * lg;
    const f4 be = *reinterpret_cast<const f4*>(&rc.beta[c]);
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = be[e] * ((float)loc.v[vb][c + e][dv] - x[e]);
    loc.x[i][db][l] = x;
  }
  phase_barrier();

  // ---- phase 2: block forward substitution (waves 0,1); most of the next record's copy (2..7)
  l = opaque(l);
  lr = l & 15, lg = l >> 4;
  // values of the next chunk into the other slot (chunk ci - 1 has read it; read after the next
  // chunk's opening barrier), before any copy is issued: waiting for them waits for nothing else
  if (more && tid < 256) *reinterpret_cast<h8*>(&loc.v[vb ^ 1][tid >> 2][8 * (tid & 3)]) = bf8_to_h8(vv);
  if (w >= 2 && more) fetch_blocks(nx, next, w - 2, kSplit, NTH / 64 - 2, l);
  if (w < 2) {
    const int dv = 16 * w + lr;
    h4 an[6], tdf[4];
    f4 X[4];
#pragma unroll
    for (int i = 0, m = 0; i < 4; ++i) {
      X[i] = loc.x[i][w][l];
      tdf[i] = frag4(&rc.td[i][0][0], 16, 0, 0, l);
#pragma unroll
      for (int j = 0; j < i; ++j, ++m) an[m] = frag4(&rc.an[m][0][0], 16, 0, 0, l);
    }
    h4 Uh[4];
#pragma unroll
    for (int i = 0, m = 0; i < 4; ++i) {
      f4 acc = X[i];
#pragma unroll
      for (int j = 0; j < i; ++j, ++m) acc = mfma16(an[m], Uh[j], acc);
      Uh[i] = to_h4(mfma16(tdf[i], to_h4(acc), f4{0.f, 0.f, 0.f, 0.f}));
      *reinterpret_cast<h4*>(sat<C>(&loc.u[0][0], dv, 16 * i + 4 * lg)) = Uh[i];
    }
  }
  phase_barrier();

  // ---- phase 3: O += U^T P^T, output (waves 2..7); S <- S Diag(Gamma_63) + U^T (K e^{G_63 - G})
  l = opaque(l);
  lr = l & 15, lg = l >> 4;
  {
    TOut* O = static_cast<TOut*>(p.o);
    const int cb = w >> 1, db = w & 1;
    f4 acc = oa;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      if (kc == 1 && cb < 2) continue;
      acc = mfma32(sfrag8<C>(&loc.u[0][0], 16 * db, 32 * kc, l), sfrag8<C>(&rc.p[0][0], 16 * cb, 32 * kc, l), acc);
    }
    const int c = 16 * cb + lr;
    if (c < n) store_o4<TOut>(O, (bh * T + t0 + c) * D + c0 + 16 * db + 4 * lg, acc);
  }
  {
    // The snapshot store goes through a buffer descriptor whose range is empty when no snapshot
    // is due, so the phase has no branch (a branch here makes the compiler wait for the copy).
    const bool snap = p.s_ckpt && n == C && ((t0 + n) % p.ckpt_every) == 0;
    const int64_t idx = snap ? (t0 + n) / p.ckpt_every - 1 : 0;
    const auto snr = __builtin_amdgcn_make_buffer_rsrc(
        snap ? (void*)(p.s_ckpt + ((bh * p.n_ckpt + idx) * D + c0) * D) : (void*)p.o, 0, snap ? DVT * D * 4 : 0,
        kRsrcWord3);
    const int dk = 16 * w + 4 * lg;
    const f4 gcv = *reinterpret_cast<const f4*>(&rc.gc[dk]);
    // every operand is read before the first LDS write of the phase (an LDS read after an LDS
    // write would make the compiler wait for the copy in flight)
    h8 ka[2], uf[2][2];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      ka[kc] = sfrag8<C>(&rc.kt[0][0], 16 * w, 32 * kc, l);
#pragma unroll
      for (int db = 0; db < 2; ++db) uf[db][kc] = sfrag8<C>(&loc.u[0][0], 16 * db, 32 * kc, l);
    }
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      f4 acc = S[db] * gcv;
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) acc = mfma32(ka[kc], uf[db][kc], acc);
      S[db] = acc;
      const int dv = 16 * db + lr;
      *reinterpret_cast<h4*>(sat<D>(&loc.s[0][0], dv, dk)) = to_h4(acc);
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, acc), snr, (dv * D + dk) * 4, 0, 0);
    }
  }
  if (w < 2 && more) fetch_blocks(nx, next, kSplit + w, kRecKiB, 2, l);
}

template <typename TOut>
__global__ __launch_bounds__(NTH, 1) void kda_chain_kernel(ChunkArgs p, const uint8_t* ws, Slab sl) {
  __shared__ KdaRec rec0;
  __shared__ KdaRec rec1;
  __shared__ ChainLocal loc;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63;

  const unsigned nblk = gridDim.x;
  unsigned bid = blockIdx.x;
  if (nblk % (8 * NT) == 0) bid = (bid % 8) * (nblk / 8) + bid / 8;
  const int c0 = (int)(bid % NT) * DVT;
  const int64_t rb = bid / NT, bh = sl.bh0 + rb;  // stream of the slab, and of the batch
  const int64_t cfirst = sl.c0, cend = sl.c0 + sl.nc;

  f4 S[2];  // wavefront w: S^T tiles (d_k block w, d_v block db)
  {
    const int lr = l & 15, lg = l >> 4;
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const int dk = 16 * w + 4 * lg, dv = 16 * db + lr;
      f4 x = {0.f, 0.f, 0.f, 0.f};
      if (sl.s_in) x = *reinterpret_cast<const f4*>(sl.s_in + (rb * D + c0 + dv) * D + dk);
      S[db] = x;
      *reinterpret_cast<h4*>(sat<D>(&loc.s[0][0], dv, dk)) = to_h4(x);
    }
  }

  const Streams sr = make_streams(p, bh, false);
  const uint8_t* recs = ws + rb * sl.nc * kRecBytes;
  v4u vv = {0u, 0u, 0u, 0u};
  if (sl.nc > 0) {
    if (tid < 256)
      vv = __builtin_amdgcn_raw_buffer_load_b128(sr.v, (int)(((cfirst * C + (tid >> 2)) * D + c0 + 8 * (tid & 3)) * 2), 0, 0);
    fetch_blocks(rec0, recs, w, kRecKiB, NTH / 64, l);
    if (tid < 256) *reinterpret_cast<h8*>(&loc.v[0][tid >> 2][8 * (tid & 3)]) = bf8_to_h8(vv);
  }
  for (int64_t ci = cfirst; ci < cend; ci += 2) {  // buffers by chunk parity; the bounds are uniform
    chain_chunk<TOut>(rec0, rec1, loc, 0, p, sr, recs, ci, cfirst, cend, bh, c0, tid, w, l, S, vv);
    if (ci + 1 < cend)
      chain_chunk<TOut>(rec1, rec0, loc, 1, p, sr, recs, ci + 1, cfirst, cend, bh, c0, tid, w, l, S, vv);
  }

  if (sl.s_out) {
    const int lr = l & 15, lg = l >> 4;
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const int dk = 16 * w + 4 * lg, dv = 16 * db + lr;
      *reinterpret_cast<f4*>(sl.s_out + (rb * D + c0 + dv) * D + dk) = S[db];
    }
  }
}

}  // namespace

size_t kda_workspace_bytes(const ChunkArgs& a) {
  const int64_t nchunks = (a.T + C - 1) / C;
  return (size_t)(a.B * a.H * nchunks) * (size_t)kRecBytes;
}

// Slab shape for a workspace of `bytes`: every record of the call when they all fit (one slab);
// otherwise as many streams as leave room for at least one chunk each plus their carried states,
// and as many chunks as then fit.
static void kda_slab_shape(int64_t streams, int64_t nchunks, size_t bytes, int64_t& nbh, int64_t& nc) {
  const int64_t slots = (int64_t)(bytes / (size_t)kRecBytes);
  if (streams * nchunks <= slots) {
    nbh = streams;
    nc = nchunks;
    return;
  }
  nbh = streams * 2 <= slots ? streams : slots / 2;  // each stream: >= 1 record and its state
  nc = slots / nbh - 1;
  if (nc > nchunks) nc = nchunks;
}

// Device scratch of the allocation-free entry point (kda_chunk_fwd_noalloc): the two-kernel
// form's records and carried states, slab by slab.  Each GPU the library runs on holds one copy
// from the first launch until the process ends.  Calls that overlap on one GPU share it and race.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
constexpr int kMaxDevices = 64;

hipError_t kda_scratch(void** ptr, size_t* bytes) {
  // The array's name is a host-side stand-in: its device address comes from the runtime, once
  // per device, with that device current.
  static std::mutex mu;
  static void* addr[kMaxDevices];
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  *bytes = kScratchBytes;
  return hipSuccess;
}

bool kda_slabs_fit(const ChunkArgs& a, size_t bytes) { return bytes / (size_t)kRecBytes >= 2 || kda_workspace_bytes(a) <= bytes; }

hipError_t launch_kda_mfma(const ChunkArgs& a, hipStream_t s) {
  const int64_t blocks = a.B * a.H * NT;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const int64_t nchunks = (a.T + C - 1) / C, streams = a.B * a.H;
  const bool two = a.workspace && nchunks > 0 && kda_slabs_fit(a, a.workspace_bytes);
  if (!two) {
    if (a.out_dtype == GDN_BF16)
      hipLaunchKernelGGL((kda_chunk_mfma_kernel<__hip_bfloat16>), dim3((unsigned)blocks), dim3(NTH), 0, s, a);
    else
      hipLaunchKernelGGL((kda_chunk_mfma_kernel<float>), dim3((unsigned)blocks), dim3(NTH), 0, s, a);
    return hipGetLastError();
  }
  // Two-kernel form, slab by slab: for each group of streams, its chunks in order, the state
  // carried from one slab to the next in the workspace after the slab's records.
  int64_t nbh, nc;
  kda_slab_shape(streams, nchunks, a.workspace_bytes, nbh, nc);
  uint8_t* ws = static_cast<uint8_t*>(a.workspace);
  float* carry = reinterpret_cast<float*>(ws + (size_t)(nbh * nc) * (size_t)kRecBytes);
  for (int64_t bh0 = 0; bh0 < streams; bh0 += nbh) {
    const int64_t ns = streams - bh0 < nbh ? streams - bh0 : nbh;
    for (int64_t c0 = 0; c0 < nchunks; c0 += nc) {
      Slab sl;
      sl.bh0 = bh0;
      sl.nbh = ns;
      sl.c0 = c0;
      sl.nc = nchunks - c0 < nc ? nchunks - c0 : nc;
      const bool first = c0 == 0, last = c0 + sl.nc >= nchunks;
      sl.s_in = first ? (a.s0 ? a.s0 + bh0 * a.D * a.D : nullptr) : carry;
      sl.s_out = last ? (a.s_final ? a.s_final + bh0 * a.D * a.D : nullptr) : carry;
      const int64_t recs = ns * sl.nc;
      // one workgroup per CU, each walking every 256th record
      const int64_t grid = recs < 256 ? recs : 256;
      hipLaunchKernelGGL(kda_prep_kernel, dim3((unsigned)grid), dim3(NTH), 0, s, a, ws, sl);
      if (a.out_dtype == GDN_BF16)
        hipLaunchKernelGGL((kda_chain_kernel<__hip_bfloat16>), dim3((unsigned)(ns * NT)), dim3(NTH), 0, s, a,
                           (const uint8_t*)ws, sl);
      else
        hipLaunchKernelGGL((kda_chain_kernel<float>), dim3((unsigned)(ns * NT)), dim3(NTH), 0, s, a,
                           (const uint8_t*)ws, sl);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace gdn
