// el_mfma.hpp -- MFMA helpers shared by the interaction kernels (gfx950 / CDNA4 only).
#pragma once

#include "el_internal.hpp"

namespace el {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Native 4 x 32-bit vector (kept in registers by the optimiser, unlike HIP's uint4 class).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Streaming 16-byte load (non-temporal): for rows that a kernel reads once and no later
// kernel needs from the cache.
__device__ inline u32x4 ld_stream16(const void* p) { return __builtin_nontemporal_load(static_cast<const u32x4*>(p)); }

template <class IT>
__device__ inline f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c);
template <>
__device__ inline f32x16 mfma32<BF16T>(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <>
__device__ inline f32x16 mfma32<F16T>(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Output row of the 32x32 MFMA accumulator: register r of lane l holds row
// 8*(r/4) + 4*(l/32) + r%4 and column l%32.
__device__ inline int acc_row(int r, int lane) { return (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3); }

// 16 bytes of LDS at `off`, or zeros when !ok (the read itself stays in bounds).
__device__ inline u32x4 lds16_or_zero(const char* lds, int off, bool ok) {
  const u32x4 v = *reinterpret_cast<const u32x4*>(lds + (ok ? off : 0));
  return ok ? v : u32x4{0, 0, 0, 0};
}

// The strict lower triangle of the Gram matrix Z = V V^T of the V x D tile at `lds` (16-bit
// elements of IT, row pitch `pitch` bytes), converted to OT and written into the staged
// output row at lds + obase: Z_ij (i > j) at element D + i(i-1)/2 + j.  One wavefront:
// the lower-triangular 32 x 32 tiles (I, J) are v_mfma_f32_32x32x16 products over K = D
// in steps of 16 (fp32 accumulate); tile entries outside the triangle or past V are
// written to the 2-byte scratch slot at `trash`.
template <class IT, class OT>
__device__ inline void gram_lower_to_lds(char* lds, int pitch, int V, int D, int obase, int trash) {
  using OS = typename OT::S;
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5, col = lane & 31;
  const int NT = (V + 31) / 32;
  for (int I = 0; I < NT; ++I) {
    for (int J = 0; J <= I; ++J) {
      f32x16 acc = {};
      const int ra = I * 32 + col, rb = J * 32 + col;
      for (int ks = 0; ks < D / 16; ++ks) {
        const int cb = (2 * ks + half) * 16;  // byte offset of this lane's 8 elements
        const u32x4 a = lds16_or_zero(lds, ra * pitch + cb, ra < V);
        const u32x4 bv = (I == J) ? a : lds16_or_zero(lds, rb * pitch + cb, rb < V);
        acc = mfma32<IT>(a, bv, acc);
      }
      const int j = J * 32 + col;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int i = I * 32 + acc_row(rr, lane);
        const int off = (i < V && j < i) ? obase + (D + i * (i - 1) / 2 + j) * static_cast<int>(sizeof(OS)) : trash;
        *reinterpret_cast<OS*>(lds + off) = OT::from_f(acc[rr]);
      }
    }
  }
}

}  // namespace el
