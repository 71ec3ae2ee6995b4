// dot_interact.hip -- pairwise "dot interaction" forward and backward (gfx950).
//
// Page "DLRM For PyTorch", §Model architecture: the bottom-MLP output and the embedding
// vectors of a sample are fed to a dot interaction, whose output is concatenated with the
// bottom-MLP output.  With V = F+1 vectors per sample (vector 0 = x0[b], vector 1+t = the
// pooled embedding of table t) the interaction is the strict lower triangle of the Gram
// matrix Z = V V^T, stored row-major: pair (i, j), i > j, at p(i,j) = i(i-1)/2 + j.
//
// 16-bit inputs (bf16 / fp16): one wavefront per sample.  The sample's V x D tile is
// streamed from HBM with 16-byte loads into LDS (row pitch padded by 16 bytes so that the
// 32 rows read by one MFMA operand fall on distinct banks), then
//   forward : the lower-triangular 32x32 tiles of Z are v_mfma_f32_32x32x16_{bf16,f16}
//             products of the tile with itself, K = D in steps of 16 (fp32 accumulate);
//   backward: dV = S V with the symmetric pair-gradient matrix S, as MFMA products of S
//             (rebuilt from the staged gradient row) and V (read transposed from LDS).
// The contraction index of each MFMA is assigned the same way in both operands, so the
// result does not depend on how the hardware orders K inside one instruction.
// fp32 inputs (and shapes the MFMA path does not cover) use an fp32 FMA kernel.
#include <algorithm>

#include "el_internal.hpp"

namespace el {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <class IT>
__device__ inline f32x16 mfma32(const uint4& a, const uint4& b, const f32x16& c);
template <>
__device__ inline f32x16 mfma32<BF16T>(const uint4& a, const uint4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <>
__device__ inline f32x16 mfma32<F16T>(const uint4& a, const uint4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

__device__ inline int64_t pair_pos(int i, int j) { return static_cast<int64_t>(i) * (i - 1) / 2 + j; }

// Output row of the 32x32 MFMA accumulator: register r of lane l holds row
// 8*(r/4) + 4*(l/32) + r%4 and column l%32.
__device__ inline int acc_row(int r, int lane) { return (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3); }

// Stage sample b's vectors (x0[b], emb[b][0..F)) into LDS rows of `pitch` bytes.  16-bit
// storage only.  Lanes holding row 0 also return it so that the caller can copy x0 out.
__device__ inline void stage_tile16(const uint16_t* __restrict__ x0, const uint16_t* __restrict__ emb,
                                    int b, int F, int D, char* lds, int pitch) {
  const int V = F + 1;
  const int nv = D / 8;
  const int lane = threadIdx.x;
  for (int q = lane; q < V * nv; q += 64) {
    const int row = q / nv, c = q - row * nv;
    const uint16_t* src = row == 0 ? x0 + static_cast<int64_t>(b) * D + c * 8
                                   : emb + (static_cast<int64_t>(b) * F + row - 1) * D + c * 8;
    *reinterpret_cast<uint4*>(lds + row * pitch + c * 16) = *reinterpret_cast<const uint4*>(src);
  }
}

// ---------------------------------------------------------------------------------------
// Forward, MFMA path.
// ---------------------------------------------------------------------------------------
template <class IT, class OT>
__global__ __launch_bounds__(64) void k_dot_fwd_mfma(const uint16_t* __restrict__ x0,
                                                     const uint16_t* __restrict__ emb, int B, int F,
                                                     int D, typename OT::S* __restrict__ out,
                                                     int out_stride) {
  extern __shared__ uint4 smem[];
  char* lds = reinterpret_cast<char*>(smem);
  const int V = F + 1;
  const int64_t P = static_cast<int64_t>(V) * (V - 1) / 2;
  const int pitch = D * 2 + 16;
  const int NT = (V + 31) / 32;
  const int lane = threadIdx.x;
  const int half = lane >> 5, col = lane & 31;

  for (int b = blockIdx.x; b < B; b += gridDim.x) {
    stage_tile16(x0, emb, b, F, D, lds, pitch);
    __syncthreads();
    typename OT::S* orow = out + static_cast<int64_t>(b) * out_stride;
    // x0 copy (converted to the output type; exact when the types agree)
    for (int d = lane; d < D; d += 64)
      orow[d] = OT::from_f(IT::to_f(*reinterpret_cast<const uint16_t*>(lds + d * 2)));
    for (int I = 0; I < NT; ++I) {
      for (int J = 0; J <= I; ++J) {
        f32x16 acc = {};
        const int ra = I * 32 + col, rb = J * 32 + col;
        for (int ks = 0; ks < D / 16; ++ks) {
          const int cb = (2 * ks + half) * 16;  // byte offset of this lane's 8 elements
          const uint4 a = ra < V ? *reinterpret_cast<const uint4*>(lds + ra * pitch + cb) : uint4{0, 0, 0, 0};
          const uint4 bv = (I == J) ? a
                           : (rb < V ? *reinterpret_cast<const uint4*>(lds + rb * pitch + cb) : uint4{0, 0, 0, 0});
          acc = mfma32<IT>(a, bv, acc);
        }
        const int j = J * 32 + col;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i = I * 32 + acc_row(r, lane);
          if (i < V && j < i) orow[D + pair_pos(i, j)] = OT::from_f(acc[r]);
        }
      }
    }
    for (int64_t c = D + P + lane; c < out_stride; c += 64) orow[c] = OT::from_f(0.0f);
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------------
// Backward, MFMA path.  dout must have the input's 16-bit type, so that S is exact.
// ---------------------------------------------------------------------------------------
template <class IT, class GT>
__global__ __launch_bounds__(64) void k_dot_bwd_mfma(const uint16_t* __restrict__ x0,
                                                     const uint16_t* __restrict__ emb, int B, int F,
                                                     int D, const uint16_t* __restrict__ dout,
                                                     int out_stride, typename GT::S* __restrict__ dx0,
                                                     typename GT::S* __restrict__ demb) {
  extern __shared__ uint4 smem[];
  char* lds = reinterpret_cast<char*>(smem);
  const int V = F + 1;
  const int64_t P = static_cast<int64_t>(V) * (V - 1) / 2;
  const int pitch = D * 2 + 16;
  uint16_t* G = reinterpret_cast<uint16_t*>(lds + V * pitch);
  const int NT = (V + 31) / 32;
  const int KS = (V + 15) / 16;
  const int lane = threadIdx.x;
  const int half = lane >> 5, col = lane & 31;
  const int64_t used = D + P;

  for (int b = blockIdx.x; b < B; b += gridDim.x) {
    stage_tile16(x0, emb, b, F, D, lds, pitch);
    const uint16_t* grow = dout + static_cast<int64_t>(b) * out_stride;
    for (int64_t c = lane; c < used; c += 64) G[c] = grow[c];
    __syncthreads();
    for (int I = 0; I < NT; ++I) {
      const int i = I * 32 + col;
      uint4 A[8];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        uint32_t w[4] = {0, 0, 0, 0};
        if (ks < KS) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int k = ks * 16 + half * 8 + e;
            uint32_t s = 0;
            if (i < V && k < V && i != k) {
              const int hi = i > k ? i : k, lo = i > k ? k : i;
              s = G[D + pair_pos(hi, lo)];
            }
            w[e >> 1] |= s << ((e & 1) * 16);
          }
        }
        A[ks] = uint4{w[0], w[1], w[2], w[3]};
      }
      for (int N = 0; N < D / 32; ++N) {
        f32x16 acc = {};
        const int n = N * 32 + col;
        for (int ks = 0; ks < KS; ++ks) {
          uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int k = ks * 16 + half * 8 + e;
            const uint32_t v = k < V ? *reinterpret_cast<const uint16_t*>(lds + k * pitch + n * 2) : 0u;
            w[e >> 1] |= v << ((e & 1) * 16);
          }
          acc = mfma32<IT>(A[ks], uint4{w[0], w[1], w[2], w[3]}, acc);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int vi = I * 32 + acc_row(r, lane);
          if (vi == 0) {
            dx0[static_cast<int64_t>(b) * D + n] = GT::from_f(IT::to_f(G[n]) + acc[r]);
          } else if (vi < V) {
            demb[(static_cast<int64_t>(b) * F + vi - 1) * D + n] = GT::from_f(acc[r]);
          }
        }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------------
// fp32 FMA path (any dtypes): one wavefront per sample, vectors staged as fp32 in LDS.
// ---------------------------------------------------------------------------------------
template <class IT>
__device__ inline void stage_tile_f32(const typename IT::S* __restrict__ x0,
                                      const typename IT::S* __restrict__ emb, int b, int F, int D,
                                      float* lv) {
  const int V = F + 1;
  for (int q = threadIdx.x; q < V * D; q += 64) {
    const int row = q / D, d = q - row * D;
    const typename IT::S v = row == 0 ? x0[static_cast<int64_t>(b) * D + d]
                                      : emb[(static_cast<int64_t>(b) * F + row - 1) * D + d];
    lv[q] = IT::to_f(v);
  }
}

template <class IT, class OT>
__global__ __launch_bounds__(64) void k_dot_fwd_valu(const typename IT::S* __restrict__ x0,
                                                     const typename IT::S* __restrict__ emb, int B,
                                                     int F, int D, typename OT::S* __restrict__ out,
                                                     int out_stride) {
  extern __shared__ uint4 smem[];
  float* lv = reinterpret_cast<float*>(smem);
  const int V = F + 1;
  const int64_t P = static_cast<int64_t>(V) * (V - 1) / 2;
  for (int b = blockIdx.x; b < B; b += gridDim.x) {
    stage_tile_f32<IT>(x0, emb, b, F, D, lv);
    __syncthreads();
    typename OT::S* orow = out + static_cast<int64_t>(b) * out_stride;
    for (int d = threadIdx.x; d < D; d += 64) orow[d] = OT::from_f(lv[d]);
    // walk pairs in row-major order; lane p handles pairs p, p+64, ...
    int i = 1, j = 0;
    int64_t p = 0;
    for (int64_t target = threadIdx.x; target < P; target += 64) {
      while (p < target) {  // advance (i, j) to pair number `target`
        ++p;
        if (++j == i) { ++i; j = 0; }
      }
      float s = 0.0f;
      for (int d = 0; d < D; ++d) s = fmaf(lv[i * D + d], lv[j * D + d], s);
      orow[D + p] = OT::from_f(s);
    }
    for (int64_t c = D + P + threadIdx.x; c < out_stride; c += 64) orow[c] = OT::from_f(0.0f);
    __syncthreads();
  }
}

template <class IT, class DT, class GT>
__global__ __launch_bounds__(64) void k_dot_bwd_valu(const typename IT::S* __restrict__ x0,
                                                     const typename IT::S* __restrict__ emb, int B,
                                                     int F, int D, const typename DT::S* __restrict__ dout,
                                                     int out_stride, typename GT::S* __restrict__ dx0,
                                                     typename GT::S* __restrict__ demb) {
  extern __shared__ uint4 smem[];
  float* lv = reinterpret_cast<float*>(smem);
  const int V = F + 1;
  const int64_t P = static_cast<int64_t>(V) * (V - 1) / 2;
  float* G = lv + V * D;
  for (int b = blockIdx.x; b < B; b += gridDim.x) {
    stage_tile_f32<IT>(x0, emb, b, F, D, lv);
    const typename DT::S* grow = dout + static_cast<int64_t>(b) * out_stride;
    for (int64_t c = threadIdx.x; c < D + P; c += 64) G[c] = DT::to_f(grow[c]);
    __syncthreads();
    for (int q = threadIdx.x; q < V * D; q += 64) {
      const int k = q / D, d = q - k * D;
      float acc = 0.0f;
      for (int j = 0; j < V; ++j) {
        if (j == k) continue;
        const int hi = j > k ? j : k, lo = j > k ? k : j;
        acc = fmaf(G[D + pair_pos(hi, lo)], lv[j * D + d], acc);
      }
      if (k == 0)
        dx0[static_cast<int64_t>(b) * D + d] = GT::from_f(G[d] + acc);
      else
        demb[(static_cast<int64_t>(b) * F + k - 1) * D + d] = GT::from_f(acc);
    }
    __syncthreads();
  }
}

constexpr size_t kMaxLds = 64 * 1024;

int grid_for(int B, size_t lds_bytes) {
  // enough one-wave workgroups to fill 256 CUs several times over; each loops over samples
  const int per_cu = lds_bytes ? static_cast<int>(std::min<size_t>(16, (160 * 1024) / lds_bytes)) : 16;
  const int g = 256 * (per_cu > 0 ? per_cu : 1);
  return B < g ? B : g;
}

template <class IT, class OT>
el_status fwd_typed(const void* x0, const void* emb, int B, int F, int D, void* out, int out_stride,
                    hipStream_t stream) {
  const int V = F + 1;
  if constexpr (sizeof(typename IT::S) == 2) {
    const size_t lds = static_cast<size_t>(V) * (D * 2 + 16);
    if (D % 16 == 0 && V <= 128 && lds <= kMaxLds) {
      hipLaunchKernelGGL((k_dot_fwd_mfma<IT, OT>), dim3(grid_for(B, lds)), dim3(64), lds, stream,
                         static_cast<const uint16_t*>(x0), static_cast<const uint16_t*>(emb), B, F, D,
                         static_cast<typename OT::S*>(out), out_stride);
      return check_launch("dot_interact_fwd");
    }
  }
  const size_t lds = static_cast<size_t>(V) * D * 4;
  if (lds > kMaxLds)
    return set_error(EL_ERR_UNSUPPORTED, "dot_interact_fwd: (F+1)*D too large for one LDS tile");
  hipLaunchKernelGGL((k_dot_fwd_valu<IT, OT>), dim3(grid_for(B, lds)), dim3(64), lds, stream,
                     static_cast<const typename IT::S*>(x0), static_cast<const typename IT::S*>(emb),
                     B, F, D, static_cast<typename OT::S*>(out), out_stride);
  return check_launch("dot_interact_fwd");
}

template <class IT, class DT, class GT>
el_status bwd_typed(const void* x0, const void* emb, int B, int F, int D, const void* dout,
                    int out_stride, void* dx0, void* demb, hipStream_t stream) {
  const int V = F + 1;
  const int64_t P = static_cast<int64_t>(V) * (V - 1) / 2;
  if constexpr (sizeof(typename IT::S) == 2 && IT::code == DT::code) {
    const size_t lds = static_cast<size_t>(V) * (D * 2 + 16) + ((D + P) * 2 + 15) / 16 * 16;
    if (D % 32 == 0 && V <= 128 && lds <= kMaxLds) {
      hipLaunchKernelGGL((k_dot_bwd_mfma<IT, GT>), dim3(grid_for(B, lds)), dim3(64), lds, stream,
                         static_cast<const uint16_t*>(x0), static_cast<const uint16_t*>(emb), B, F, D,
                         static_cast<const uint16_t*>(dout), out_stride,
                         static_cast<typename GT::S*>(dx0), static_cast<typename GT::S*>(demb));
      return check_launch("dot_interact_bwd");
    }
  }
  const size_t lds = (static_cast<size_t>(V) * D + D + P) * 4;
  if (lds > kMaxLds)
    return set_error(EL_ERR_UNSUPPORTED, "dot_interact_bwd: (F+1)*D + pairs too large for LDS");
  hipLaunchKernelGGL((k_dot_bwd_valu<IT, DT, GT>), dim3(grid_for(B, lds)), dim3(64), lds, stream,
                     static_cast<const typename IT::S*>(x0), static_cast<const typename IT::S*>(emb),
                     B, F, D, static_cast<const typename DT::S*>(dout), out_stride,
                     static_cast<typename GT::S*>(dx0), static_cast<typename GT::S*>(demb));
  return check_launch("dot_interact_bwd");
}

// dtype dispatch helpers
template <class F>
el_status with_type(el_dtype d, F&& f) {
  switch (d) {
    case EL_F32: return f(F32T{});
    case EL_F16: return f(F16T{});
    case EL_BF16: return f(BF16T{});
  }
  return set_error(EL_ERR_INVALID_ARG, "unknown dtype");
}

}  // namespace

el_status launch_dot_fwd(const void* x0, const void* emb, el_dtype in_dtype, int B, int F, int D,
                         void* out, el_dtype out_dtype, int out_stride, hipStream_t stream) {
  return with_type(in_dtype, [&](auto it) {
    return with_type(out_dtype, [&](auto ot) {
      return fwd_typed<decltype(it), decltype(ot)>(x0, emb, B, F, D, out, out_stride, stream);
    });
  });
}

el_status launch_dot_bwd(const void* x0, const void* emb, el_dtype in_dtype, int B, int F, int D,
                         const void* dout, el_dtype dout_dtype, int out_stride, void* dx0,
                         void* demb, el_dtype grad_dtype, hipStream_t stream) {
  return with_type(in_dtype, [&](auto it) {
    return with_type(dout_dtype, [&](auto dt) {
      return with_type(grad_dtype, [&](auto gt) {
        return bwd_typed<decltype(it), decltype(dt), decltype(gt)>(x0, emb, B, F, D, dout, out_stride,
                                                                   dx0, demb, stream);
      });
    });
  });
}

}  // namespace el
