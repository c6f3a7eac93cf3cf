// gdn_mfma_common.h -- device helpers shared by the matrix-core prefill kernels (gfx950):
// fragment loads in the MFMA operand layouts, half-precision conversions, the DPP wave
// prefix sum and the output store.  Internal to libgdn.so.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>

namespace gdn {
namespace mfma {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f4 mfma32(h8 a, h8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 mfma16(h4 a, h4 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

// Returns x unchanged but opaque to the optimiser, so per-lane addresses derived from it are
// recomputed where they are used instead of being hoisted out of the chunk loop and kept
// live across every phase.
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

// A transposed tile [channel][token] stores its 16-byte groups of 8 tokens XOR-swizzled
// by bits 3..5 of the key channel, so that the staging writes (16 lanes writing 16 channels
// 8 apart, same tokens) spread over the LDS banks; 16-byte reads stay contiguous.
__device__ __forceinline__ int kt_col(int dk, int c) { return (((c >> 3) ^ ((dk >> 3) & 7)) << 3) | (c & 7); }

// Two accumulator-layout 16x16 tiles t0 (rows 0..15) and t1 (rows 16..31) of a 32-row block,
// rounded to fp16, regrouped in registers into the 16x16x32 operand layout in which the 32
// rows are the contraction index: lane (column c, group g) receives rows 8g .. 8g+7 of
// column c.  In a tile, lane group g holds rows 4g .. 4g+3; per dword, one permlane32 swap
// and one permlane16 swap (gfx950) bring them to the lane groups that need them:
//   (A0 A1 A2 A3), (B0 B1 B2 B3) -> (A0 A1 B0 B1), (A2 A3 B2 B3) -> (A0 A2 B0 B2), (A1 A3 B1 B3)
// where Xg is the value of lane group g; the first result holds rows 8g..8g+3, the second
// rows 8g+4..8g+7.
__device__ __forceinline__ h8 pair_k32(h4 t0, h4 t1) {
  typedef unsigned u2 __attribute__((ext_vector_type(2)));
  const u2 a = __builtin_bit_cast(u2, t0), b = __builtin_bit_cast(u2, t1);
  v4u r;
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    const u2 s32 = __builtin_amdgcn_permlane32_swap(a[d], b[d], false, false);
    const u2 s16 = __builtin_amdgcn_permlane16_swap(s32[0], s32[1], false, false);
    r[d] = s16[0];
    r[2 + d] = s16[1];
  }
  return __builtin_bit_cast(h8, r);
}

__device__ __forceinline__ h4 to_h4(f4 x) {
  h4 r;
  r[0] = (_Float16)x[0]; r[1] = (_Float16)x[1]; r[2] = (_Float16)x[2]; r[3] = (_Float16)x[3];
  return r;
}

// 8 bf16 (packed in 4 dwords, element 2i in the low half) -> 8 fp16.  bf16 -> fp16 is exact
// for |x| in [2^-14, 65504] (8 significant bits fit in 11), so the round-toward-zero packed
// conversion gives the same bits as round-to-nearest at 3 instructions per pair.
__device__ __forceinline__ h8 bf8_to_h8(v4u x) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  h8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const h2 pr = __builtin_bit_cast(
        h2, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(x[i] << 16), __uint_as_float(x[i] & 0xffff0000u)));
    r[2 * i] = pr[0];
    r[2 * i + 1] = pr[1];
  }
  return r;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const uint32_t lo = __bfloat16_as_ushort(__float2bfloat16(a));
  const uint32_t hi = __bfloat16_as_ushort(__float2bfloat16(b));
  return lo | (hi << 16);
}

// Inclusive prefix sum over the 64 lanes of a wavefront with DPP: shifts within rows of 16
// lanes, then the row broadcasts of lane 15 and lane 31.
__device__ __forceinline__ float wave_prefix_sum(float x) {
  int v = __float_as_int(x);
#define GDN_DPP_STEP(ctrl, rows) \
  v = __float_as_int(__int_as_float(v) + __int_as_float(__builtin_amdgcn_update_dpp(0, v, ctrl, rows, 0xf, false)))
  GDN_DPP_STEP(0x111, 0xf);  // row_shr:1
  GDN_DPP_STEP(0x112, 0xf);  // row_shr:2
  GDN_DPP_STEP(0x114, 0xf);  // row_shr:4
  GDN_DPP_STEP(0x118, 0xf);  // row_shr:8
  GDN_DPP_STEP(0x142, 0xa);  // row_bcast:15 into rows 1 and 3
  GDN_DPP_STEP(0x143, 0xc);  // row_bcast:31 into rows 2 and 3
#undef GDN_DPP_STEP
  return __int_as_float(v);
}


// gfx9-family raw buffer descriptor word 3: 32-bit dwords, no swizzle.
constexpr int kRsrcWord3 = 0x00020000;

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

}  // namespace mfma
}  // namespace gdn
