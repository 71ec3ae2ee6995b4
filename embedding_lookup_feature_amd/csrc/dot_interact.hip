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

// Native 4 x 32-bit vector (kept in registers by the optimiser, unlike HIP's uint4 class).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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

__device__ inline int64_t pair_pos(int i, int j) { return static_cast<int64_t>(i) * (i - 1) / 2 + j; }

// Output row of the 32x32 MFMA accumulator: register r of lane l holds row
// 8*(r/4) + 4*(l/32) + r%4 and column l%32.
__device__ inline int acc_row(int r, int lane) { return (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3); }

// One sample's inputs as a sequence of 16-byte chunks, lane-strided over the wavefront:
// chunks [0, tile) are the V x D tile (row 0 = x0[b], rows 1.. = emb[b], contiguous in
// memory), chunks [tile, total) the first elements of the upstream-gradient row
// (backward only).  All of a sample's loads are issued back to back into registers; the
// caller issues the next sample's loads before computing on the current one, so one
// sample's HBM latency hides behind the previous sample's MFMA work.  Lanes past the end
// re-load the last chunk (in bounds, no branch) and later write it to a scratch LDS slot.
template <int NQ, bool WITH_GRAD>
__device__ inline void fetch_sample(const uint16_t* __restrict__ x0, const uint16_t* __restrict__ emb,
                                    const uint16_t* __restrict__ dout, int out_stride, int b, int F,
                                    int D, int tile, int total, u32x4 (&r)[NQ]) {
  const int nv = D / 8;
  const int64_t x0_base = static_cast<int64_t>(b) * D;
  const int64_t emb_base = static_cast<int64_t>(b) * F * D - static_cast<int64_t>(nv) * 8;
  const int64_t g_base = static_cast<int64_t>(b) * out_stride - static_cast<int64_t>(tile) * 8;
#pragma unroll
  for (int u = 0; u < NQ; ++u) {
    int q = u * 64 + static_cast<int>(threadIdx.x);
    q = q < total ? q : total - 1;
    const uint16_t* src;
    if constexpr (WITH_GRAD) {
      src = q < nv ? x0 + x0_base + q * 8 : (q < tile ? emb + emb_base + q * 8 : dout + g_base + q * 8);
    } else {
      src = q < nv ? x0 + x0_base + q * 8 : emb + emb_base + q * 8;
    }
    r[u] = *reinterpret_cast<const u32x4*>(src);
  }
}

// Write the fetched chunks to LDS: tile rows at `pitch`-byte pitch from offset 0, gradient
// chunks packed from byte `goff`, chunks past the end to the scratch slot at `trash`.
template <int NQ>
__device__ inline void put_sample(char* lds, int pitch, int goff, int trash, int D, int tile,
                                  int total, const u32x4 (&r)[NQ]) {
  const int nv = D / 8;
#pragma unroll
  for (int u = 0; u < NQ; ++u) {
    const int q = u * 64 + static_cast<int>(threadIdx.x);
    const int row = q / nv, c = q - row * nv;
    const int off = q < tile ? row * pitch + c * 16 : (q < total ? goff + (q - tile) * 16 : trash);
    *reinterpret_cast<u32x4*>(lds + off) = r[u];
  }
}

__device__ inline u32x4 lds16_or_zero(const char* lds, int off, bool ok) {
  const u32x4 v = *reinterpret_cast<const u32x4*>(lds + (ok ? off : 0));
  return ok ? v : u32x4{0, 0, 0, 0};
}

// ---------------------------------------------------------------------------------------
// Forward, MFMA path.
// LDS: V x D tile (pitch 2D+16) | one output row (16-byte rounded) | 16-byte scratch slot.
// ---------------------------------------------------------------------------------------
template <class IT, class OT, int NQ>
__global__ __launch_bounds__(64) void k_dot_fwd_mfma(const uint16_t* __restrict__ x0,
                                                     const uint16_t* __restrict__ emb, int B, int F,
                                                     int D, typename OT::S* __restrict__ out,
                                                     int out_stride, int vec_out) {
  extern __shared__ uint4 smem[];
  char* lds = reinterpret_cast<char*>(smem);
  using OS = typename OT::S;
  const int V = F + 1;
  const int P = V * (V - 1) / 2;
  const int pitch = D * 2 + 16;
  const int obase = V * pitch;
  const int obytes = (out_stride * static_cast<int>(sizeof(OS)) + 15) / 16 * 16;
  const int trash = obase + obytes;
  OS* ostage = reinterpret_cast<OS*>(lds + obase);
  const int NT = (V + 31) / 32;
  const int lane = threadIdx.x;
  const int half = lane >> 5, col = lane & 31;
  const int tile = V * (D / 8);

  u32x4 r[NQ];
  int b = blockIdx.x;
  if (b < B) fetch_sample<NQ, false>(x0, emb, x0, 0, b, F, D, tile, tile, r);
  for (; b < B; b += gridDim.x) {
    put_sample<NQ>(lds, pitch, 0, trash, D, tile, tile, r);
    if (b + static_cast<int>(gridDim.x) < B)
      fetch_sample<NQ, false>(x0, emb, x0, 0, b + gridDim.x, F, D, tile, tile, r);
    __syncthreads();
    // x0 copy (converted to the output type; exact when the types agree) and zero padding
    for (int d = lane; d < D; d += 64)
      ostage[d] = OT::from_f(IT::to_f(*reinterpret_cast<const uint16_t*>(lds + d * 2)));
    for (int c = D + P + lane; c < out_stride; c += 64) ostage[c] = OT::from_f(0.0f);
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
    __syncthreads();
    OS* orow = out + static_cast<int64_t>(b) * out_stride;
    if (vec_out) {
      for (int q = lane; q < obytes / 16; q += 64)
        reinterpret_cast<u32x4*>(orow)[q] = reinterpret_cast<const u32x4*>(ostage)[q];
    } else {
      for (int c = lane; c < out_stride; c += 64) orow[c] = ostage[c];
    }
  }
}

// ---------------------------------------------------------------------------------------
// Backward, MFMA path.  dout has the input's 16-bit type (so that S is exact) and a row
// stride that is a multiple of 8 elements (16-byte chunks of the D + P used columns stay
// inside the row).
// LDS: V x D tile | gradient row | (32*NT) x D output block (pitch D*sizeof+16) | scratch.
// ---------------------------------------------------------------------------------------
template <class IT, class GT, int NQ, int KSM>
__global__ __launch_bounds__(64) void k_dot_bwd_mfma(const uint16_t* __restrict__ x0,
                                                     const uint16_t* __restrict__ emb, int B, int F,
                                                     int D, const uint16_t* __restrict__ dout,
                                                     int out_stride, typename GT::S* __restrict__ dx0,
                                                     typename GT::S* __restrict__ demb) {
  extern __shared__ uint4 smem[];
  char* lds = reinterpret_cast<char*>(smem);
  using GS = typename GT::S;
  const int V = F + 1;
  const int P = V * (V - 1) / 2;
  const int pitch = D * 2 + 16;
  const int gchunks = (D + P + 7) / 8;
  const int goff = V * pitch;
  const uint16_t* G = reinterpret_cast<const uint16_t*>(lds + goff);
  const int NT = (V + 31) / 32;
  const int opitch = D * static_cast<int>(sizeof(GS)) + 16;
  const int ooff = goff + gchunks * 16;
  const int trash = ooff + NT * 32 * opitch;
  const int KS = (V + 15) / 16;
  const int lane = threadIdx.x;
  const int half = lane >> 5, col = lane & 31;
  const int tile = V * (D / 8);
  const int total = tile + gchunks;

  u32x4 r[NQ];
  int b = blockIdx.x;
  if (b < B) fetch_sample<NQ, true>(x0, emb, dout, out_stride, b, F, D, tile, total, r);
  for (; b < B; b += gridDim.x) {
    put_sample<NQ>(lds, pitch, goff, trash, D, tile, total, r);
    if (b + static_cast<int>(gridDim.x) < B)
      fetch_sample<NQ, true>(x0, emb, dout, out_stride, b + gridDim.x, F, D, tile, total, r);
    __syncthreads();
    for (int I = 0; I < NT; ++I) {
      const int i = I * 32 + col;
      u32x4 A[KSM];  // rows of S for the K steps of 16 vectors
#pragma unroll
      for (int ks = 0; ks < KSM; ++ks) {
        uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int k = ks * 16 + half * 8 + e;
          const bool ok = i < V && k < V && i != k;
          const int hi = i > k ? i : k, lo = i > k ? k : i;
          const uint32_t sv = G[ok ? D + hi * (hi - 1) / 2 + lo : 0];
          w[e >> 1] |= (ok ? sv : 0u) << ((e & 1) * 16);
        }
        A[ks] = u32x4{w[0], w[1], w[2], w[3]};
      }
      for (int N = 0; N < D / 32; ++N) {
        f32x16 acc = {};
        const int n = N * 32 + col;
#pragma unroll
        for (int ks = 0; ks < KSM; ++ks) {
          if (ks < KS) {
            uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int k = ks * 16 + half * 8 + e;
              const uint32_t v = *reinterpret_cast<const uint16_t*>(lds + (k < V ? k : 0) * pitch + n * 2);
              w[e >> 1] |= (k < V ? v : 0u) << ((e & 1) * 16);
            }
            acc = mfma32<IT>(A[ks], u32x4{w[0], w[1], w[2], w[3]}, acc);
          }
        }
        const float g0 = IT::to_f(G[n]);
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const int vi = I * 32 + acc_row(rr, lane);  // rows >= V land in unused output rows
          const float v = vi == 0 ? g0 + acc[rr] : acc[rr];
          *reinterpret_cast<GS*>(lds + ooff + vi * opitch + n * static_cast<int>(sizeof(GS))) = GT::from_f(v);
        }
      }
    }
    __syncthreads();
    // row 0 -> dx0[b], rows 1.. -> demb[b] (contiguous), 16-byte stores
    const int nv = D * static_cast<int>(sizeof(GS)) / 16;
    char* dxrow = reinterpret_cast<char*>(dx0 + static_cast<int64_t>(b) * D);
    char* derow = reinterpret_cast<char*>(demb + static_cast<int64_t>(b) * F * D) - nv * 16;
    for (int q = lane; q < V * nv; q += 64) {
      const int row = q / nv, c = q - row * nv;
      const u32x4 v = *reinterpret_cast<const u32x4*>(lds + ooff + row * opitch + c * 16);
      char* dst = row == 0 ? dxrow + c * 16 : derow + static_cast<int64_t>(q) * 16;
      *reinterpret_cast<u32x4*>(dst) = v;
    }
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

template <class IT, class OT, int NQ>
el_status launch_fwd_mfma(const void* x0, const void* emb, int B, int F, int D, void* out,
                          int out_stride, size_t lds, hipStream_t stream) {
  const int vec_out = (static_cast<int64_t>(out_stride) * sizeof(typename OT::S)) % 16 == 0;
  hipLaunchKernelGGL((k_dot_fwd_mfma<IT, OT, NQ>), dim3(grid_for(B, lds)), dim3(64), lds, stream,
                     static_cast<const uint16_t*>(x0), static_cast<const uint16_t*>(emb), B, F, D,
                     static_cast<typename OT::S*>(out), out_stride, vec_out);
  return check_launch("dot_interact_fwd");
}

template <class IT, class OT>
el_status fwd_typed(const void* x0, const void* emb, int B, int F, int D, void* out, int out_stride,
                    hipStream_t stream) {
  const int V = F + 1;
  if constexpr (sizeof(typename IT::S) == 2) {
    const size_t ost = (static_cast<size_t>(out_stride) * sizeof(typename OT::S) + 15) / 16 * 16;
    const size_t lds = static_cast<size_t>(V) * (D * 2 + 16) + ost + 16;
    const int chunks = V * (D / 8);
    if (D % 16 == 0 && V <= 128 && lds <= kMaxLds && chunks <= 32 * 64) {
      if (chunks <= 8 * 64) return launch_fwd_mfma<IT, OT, 8>(x0, emb, B, F, D, out, out_stride, lds, stream);
      if (chunks <= 16 * 64) return launch_fwd_mfma<IT, OT, 16>(x0, emb, B, F, D, out, out_stride, lds, stream);
      return launch_fwd_mfma<IT, OT, 32>(x0, emb, B, F, D, out, out_stride, lds, stream);
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

template <class IT, class GT, int NQ, int KSM>
el_status launch_bwd_ks(const void* x0, const void* emb, int B, int F, int D, const void* dout,
                        int out_stride, void* dx0, void* demb, size_t lds, hipStream_t stream) {
  hipLaunchKernelGGL((k_dot_bwd_mfma<IT, GT, NQ, KSM>), dim3(grid_for(B, lds)), dim3(64), lds, stream,
                     static_cast<const uint16_t*>(x0), static_cast<const uint16_t*>(emb), B, F, D,
                     static_cast<const uint16_t*>(dout), out_stride,
                     static_cast<typename GT::S*>(dx0), static_cast<typename GT::S*>(demb));
  return check_launch("dot_interact_bwd");
}

// K steps of the S V product: one per 16 vectors
template <class IT, class GT, int NQ>
el_status launch_bwd_mfma(const void* x0, const void* emb, int B, int F, int D, const void* dout,
                          int out_stride, void* dx0, void* demb, size_t lds, hipStream_t stream) {
  const int V = F + 1;
  if (V <= 32) return launch_bwd_ks<IT, GT, NQ, 2>(x0, emb, B, F, D, dout, out_stride, dx0, demb, lds, stream);
  if (V <= 64) return launch_bwd_ks<IT, GT, NQ, 4>(x0, emb, B, F, D, dout, out_stride, dx0, demb, lds, stream);
  return launch_bwd_ks<IT, GT, NQ, 8>(x0, emb, B, F, D, dout, out_stride, dx0, demb, lds, stream);
}

template <class IT, class DT, class GT>
el_status bwd_typed(const void* x0, const void* emb, int B, int F, int D, const void* dout,
                    int out_stride, void* dx0, void* demb, hipStream_t stream) {
  const int V = F + 1;
  const int64_t P = static_cast<int64_t>(V) * (V - 1) / 2;
  if constexpr (sizeof(typename IT::S) == 2 && IT::code == DT::code) {
    const int64_t gchunks = (D + P + 7) / 8;
    const size_t lds = static_cast<size_t>(V) * (D * 2 + 16) + gchunks * 16 +
                       static_cast<size_t>((V + 31) / 32 * 32) * (D * sizeof(typename GT::S) + 16) + 16;
    const int64_t chunks = static_cast<int64_t>(V) * (D / 8) + gchunks;
    // 16-byte chunks of the gradient row must stay inside the row: stride multiple of 8
    if (D % 32 == 0 && V <= 128 && lds <= kMaxLds && out_stride % 8 == 0 && chunks <= 32 * 64) {
      if (chunks <= 8 * 64)
        return launch_bwd_mfma<IT, GT, 8>(x0, emb, B, F, D, dout, out_stride, dx0, demb, lds, stream);
      if (chunks <= 16 * 64)
        return launch_bwd_mfma<IT, GT, 16>(x0, emb, B, F, D, dout, out_stride, dx0, demb, lds, stream);
      return launch_bwd_mfma<IT, GT, 32>(x0, emb, B, F, D, dout, out_stride, dx0, demb, lds, stream);
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
