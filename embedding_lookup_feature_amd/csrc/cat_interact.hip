// cat_interact.hip -- the "cat" interaction (page "DLRM For PyTorch", §Command-line options,
// --interaction_op cat) forward and backward, and its fused form with the embedding-bag
// gather (gfx950).
//
// The cat interaction puts a sample's V = F+1 vectors side by side instead of multiplying
// them: out[b] = [x0[b] | emb[b][0] | ... | emb[b][F-1] | +0 pad] (V*D values, then zeros up
// to out_stride).  The model's concatenation of the interaction output with the bottom-MLP
// output is the first block itself.  Its backward hands each vector its own block of the
// upstream gradient: dx0[b] = G[0:D), demb[b][t] = G[D(1+t) : D(2+t)).
//
// Both directions are pure data movement, priced against HBM bandwidth.  A thread moves
// 16-byte chunks of the output side (8 16-bit or 4 fp32 values), K of them in flight: all K
// loads are issued before any store.  Because D is a multiple of the chunk's element count
// on this path, a chunk never straddles two vectors or a vector and the padding.  Shapes
// where it is not (D or the row stride not a multiple of the chunk) take a one-element-per-
// thread kernel.  Conversions between dtypes round to nearest even (one rounding); equal
// dtypes copy bits.
//
// emb_cat_fwd: the gather writes each pooled vector straight into its block of the output
// row (launch_emb_bag_fwd with the output row stride), and a copy kernel writes the x0
// block and the zero padding of every row: the pooled vectors are never stored elsewhere.
#include "el_internal.hpp"

namespace el {
namespace {

constexpr int kChunksPerThread = 4;

// EV elements of T starting at p (EV * sizeof(T::S) bytes, naturally aligned) as floats.
template <class T, int EV>
__device__ inline void load_ev(const typename T::S* p, float* f) {
  constexpr int BYTES = EV * static_cast<int>(sizeof(typename T::S));
  if constexpr (BYTES == 32) {
    unpack16<T>(reinterpret_cast<const uint4*>(p)[0], f);
    unpack16<T>(reinterpret_cast<const uint4*>(p)[1], f + 16 / static_cast<int>(sizeof(typename T::S)));
  } else if constexpr (BYTES == 16) {
    unpack16<T>(*reinterpret_cast<const uint4*>(p), f);
  } else {  // 8 bytes: four 16-bit values
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    unpack16<T>(uint4{v.x, v.y, 0u, 0u}, f);
  }
}

// Raw EV-element chunk of the input side, kept as bits until it is converted (so that all
// of a thread's loads are in flight before the first conversion).
template <class T, int EV>
struct Chunk {
  static constexpr int N = (EV * static_cast<int>(sizeof(typename T::S)) + 15) / 16;  // 16-byte vectors
  uint4 v[N];
};

template <class T, int EV>
__device__ inline void load_chunk(Chunk<T, EV>& c, const typename T::S* p) {
  constexpr int BYTES = EV * static_cast<int>(sizeof(typename T::S));
  if constexpr (BYTES >= 16) {
#pragma unroll
    for (int i = 0; i < Chunk<T, EV>::N; ++i) c.v[i] = reinterpret_cast<const uint4*>(p)[i];
  } else {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    c.v[0] = uint4{v.x, v.y, 0u, 0u};
  }
}

template <class T, int EV>
__device__ inline void chunk_to_f(const Chunk<T, EV>& c, float* f) {
  constexpr int PER = 16 / static_cast<int>(sizeof(typename T::S));
#pragma unroll
  for (int i = 0; i < Chunk<T, EV>::N; ++i) {
    float g[PER];
    unpack16<T>(c.v[i], g);
#pragma unroll
    for (int x = 0; x < PER; ++x)
      if (i * PER + x < EV) f[i * PER + x] = g[x];
  }
}

// Forward, vector path.  Output chunk q of row b (EV = 16 / sizeof(OT) elements) comes from
// x0 (q < nd), from emb (q < nv) or is padding.  With skip_emb (emb_cat_fwd) the emb
// chunks are not visited: the gather writes them.  Chunk numbers are row-major over the
// visited chunks of all rows.
template <class IT, class OT>
__global__ __launch_bounds__(256) void k_cat_fwd(const typename IT::S* __restrict__ x0,
                                                 const typename IT::S* __restrict__ emb, int B,
                                                 int F, int D, typename OT::S* __restrict__ out,
                                                 int out_stride, int skip_emb) {
  constexpr int EV = 16 / static_cast<int>(sizeof(typename OT::S));
  const int nd = D / EV;                       // x0 chunks per row
  const int nv = (F + 1) * D / EV;             // x0 + emb chunks per row
  const int nq = out_stride / EV;              // chunks per output row
  const int per_row = skip_emb ? nq - (nv - nd) : nq;  // visited chunks per row
  const int64_t total = static_cast<int64_t>(B) * per_row;
  const int64_t first = (static_cast<int64_t>(blockIdx.x) * kChunksPerThread) * 256 + threadIdx.x;
  Chunk<IT, EV> in[kChunksPerThread];
  int64_t dst[kChunksPerThread];
  int kind[kChunksPerThread];  // 0: x0 or emb (loaded), 1: padding, -1: past the end
#pragma unroll
  for (int k = 0; k < kChunksPerThread; ++k) {
    const int64_t i = first + static_cast<int64_t>(k) * 256;
    kind[k] = -1;
    dst[k] = 0;
    if (i < total) {
      const int64_t b = i / per_row;
      int q = static_cast<int>(i - b * per_row);
      if (skip_emb && q >= nd) q += nv - nd;  // skip the emb chunks
      dst[k] = b * out_stride + static_cast<int64_t>(q) * EV;
      if (q < nv) {
        const typename IT::S* src = q < nd ? x0 + b * D + static_cast<int64_t>(q) * EV
                                           : emb + b * F * static_cast<int64_t>(D) + static_cast<int64_t>(q - nd) * EV;
        load_chunk<IT, EV>(in[k], src);
        kind[k] = 0;
      } else {
        kind[k] = 1;
      }
    }
  }
#pragma unroll
  for (int k = 0; k < kChunksPerThread; ++k) {
    if (kind[k] < 0) continue;
    if constexpr (IT::code == OT::code) {
      *reinterpret_cast<uint4*>(out + dst[k]) = kind[k] == 0 ? in[k].v[0] : uint4{0u, 0u, 0u, 0u};
    } else {
      float f[EV];
      if (kind[k] == 0) {
        chunk_to_f<IT, EV>(in[k], f);
      } else {
#pragma unroll
        for (int x = 0; x < EV; ++x) f[x] = 0.0f;
      }
      store_n<OT, EV>(out + dst[k], f);
    }
  }
}

// Backward, vector path.  Chunk q of the V*D gradient values of sample b (EV = 16 /
// sizeof(GT) elements) goes to dx0 (q < nd) or demb; its source is the same columns of
// dout.
template <class DT, class GT>
__global__ __launch_bounds__(256) void k_cat_bwd(const typename DT::S* __restrict__ dout, int B,
                                                 int F, int D, int out_stride,
                                                 typename GT::S* __restrict__ dx0,
                                                 typename GT::S* __restrict__ demb) {
  constexpr int EV = 16 / static_cast<int>(sizeof(typename GT::S));
  const int nd = D / EV;
  const int nv = (F + 1) * D / EV;
  const int64_t total = static_cast<int64_t>(B) * nv;
  const int64_t first = (static_cast<int64_t>(blockIdx.x) * kChunksPerThread) * 256 + threadIdx.x;
  Chunk<DT, EV> in[kChunksPerThread];
  typename GT::S* dst[kChunksPerThread];
#pragma unroll
  for (int k = 0; k < kChunksPerThread; ++k) {
    const int64_t i = first + static_cast<int64_t>(k) * 256;
    dst[k] = nullptr;
    if (i < total) {
      const int64_t b = i / nv;
      const int q = static_cast<int>(i - b * nv);
      load_chunk<DT, EV>(in[k], dout + b * out_stride + static_cast<int64_t>(q) * EV);
      dst[k] = q < nd ? dx0 + b * D + static_cast<int64_t>(q) * EV
                      : demb + b * F * static_cast<int64_t>(D) + static_cast<int64_t>(q - nd) * EV;
    }
  }
#pragma unroll
  for (int k = 0; k < kChunksPerThread; ++k) {
    if (!dst[k]) continue;
    if constexpr (DT::code == GT::code) {
      *reinterpret_cast<uint4*>(dst[k]) = in[k].v[0];
    } else {
      float f[EV];
      chunk_to_f<DT, EV>(in[k], f);
      store_n<GT, EV>(dst[k], f);
    }
  }
}

// One element per thread (any D and row stride), grid-strided.
template <class IT, class OT>
__global__ __launch_bounds__(256) void k_cat_fwd_scalar(const typename IT::S* __restrict__ x0,
                                                        const typename IT::S* __restrict__ emb,
                                                        int B, int F, int D,
                                                        typename OT::S* __restrict__ out,
                                                        int out_stride) {
  const int64_t total = static_cast<int64_t>(B) * out_stride;
  const int64_t VD = static_cast<int64_t>(F + 1) * D;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t b = i / out_stride, c = i - b * out_stride;
    float v = 0.0f;
    if (c < D) v = IT::to_f(x0[b * D + c]);
    else if (c < VD) v = IT::to_f(emb[b * F * static_cast<int64_t>(D) + c - D]);
    out[i] = OT::from_f(v);
  }
}

template <class DT, class GT>
__global__ __launch_bounds__(256) void k_cat_bwd_scalar(const typename DT::S* __restrict__ dout,
                                                        int B, int F, int D, int out_stride,
                                                        typename GT::S* __restrict__ dx0,
                                                        typename GT::S* __restrict__ demb) {
  const int64_t VD = static_cast<int64_t>(F + 1) * D;
  const int64_t total = static_cast<int64_t>(B) * VD;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t b = i / VD, c = i - b * VD;
    const typename GT::S g = GT::from_f(DT::to_f(dout[b * out_stride + c]));
    if (c < D) dx0[b * D + c] = g;
    else demb[b * F * static_cast<int64_t>(D) + c - D] = g;
  }
}

int blocks_of(int64_t items) {
  const int64_t per = static_cast<int64_t>(256) * kChunksPerThread;
  return static_cast<int>((items + per - 1) / per);
}

int scalar_grid(int64_t total) {
  const int64_t g = (total + 255) / 256;
  return static_cast<int>(g < 256 * 64 ? g : 256 * 64);
}

template <class IT, class OT>
el_status fwd_typed(const void* x0, const void* emb, int B, int F, int D, void* out,
                    int out_stride, bool skip_emb, hipStream_t stream) {
  constexpr int EV = 16 / static_cast<int>(sizeof(typename OT::S));
  using IS = typename IT::S;
  using OS = typename OT::S;
  if (D % EV == 0 && out_stride % EV == 0) {
    const int nd = D / EV, nv = (F + 1) * D / EV, nq = out_stride / EV;
    const int per_row = skip_emb ? nq - (nv - nd) : nq;
    const int64_t total = static_cast<int64_t>(B) * per_row;
    if (total == 0) return EL_OK;
    hipLaunchKernelGGL((k_cat_fwd<IT, OT>), dim3(blocks_of(total)), dim3(256), 0, stream,
                       static_cast<const IS*>(x0), static_cast<const IS*>(emb), B, F, D,
                       static_cast<OS*>(out), out_stride, skip_emb ? 1 : 0);
    return check_launch("cat_interact_fwd");
  }
  if (skip_emb) return set_error(EL_ERR_UNSUPPORTED, "emb_cat_fwd: D and out_stride must be multiples of 16 bytes of the activation type");
  hipLaunchKernelGGL((k_cat_fwd_scalar<IT, OT>), dim3(scalar_grid(static_cast<int64_t>(B) * out_stride)),
                     dim3(256), 0, stream, static_cast<const IS*>(x0), static_cast<const IS*>(emb), B,
                     F, D, static_cast<OS*>(out), out_stride);
  return check_launch("cat_interact_fwd");
}

template <class DT, class GT>
el_status bwd_typed(const void* dout, int B, int F, int D, int out_stride, void* dx0, void* demb,
                    hipStream_t stream) {
  constexpr int EV = 16 / static_cast<int>(sizeof(typename GT::S));
  using DS = typename DT::S;
  using GS = typename GT::S;
  // the input side of a chunk (EV values of DT) must be aligned to its own size
  const bool aligned = (static_cast<int64_t>(out_stride) * static_cast<int64_t>(sizeof(DS))) %
                           (EV * static_cast<int64_t>(sizeof(DS))) == 0;
  if (D % EV == 0 && aligned) {
    const int64_t total = static_cast<int64_t>(B) * ((F + 1) * D / EV);
    hipLaunchKernelGGL((k_cat_bwd<DT, GT>), dim3(blocks_of(total)), dim3(256), 0, stream,
                       static_cast<const DS*>(dout), B, F, D, out_stride, static_cast<GS*>(dx0),
                       static_cast<GS*>(demb));
    return check_launch("cat_interact_bwd");
  }
  hipLaunchKernelGGL((k_cat_bwd_scalar<DT, GT>),
                     dim3(scalar_grid(static_cast<int64_t>(B) * (F + 1) * D)), dim3(256), 0, stream,
                     static_cast<const DS*>(dout), B, F, D, out_stride, static_cast<GS*>(dx0),
                     static_cast<GS*>(demb));
  return check_launch("cat_interact_bwd");
}

template <class F>
el_status with_type(el_dtype d, F&& f) {
  switch (d) {
    case EL_F32: return f(F32T{});
    case EL_F16: return f(F16T{});
    case EL_BF16: return f(BF16T{});
    default: break;
  }
  return set_error(EL_ERR_INVALID_ARG, "unknown dtype");
}

}  // namespace

el_status launch_cat_fwd(const void* x0, const void* emb, el_dtype in_dtype, int B, int F, int D,
                         void* out, el_dtype out_dtype, int out_stride, hipStream_t stream) {
  return with_type(in_dtype, [&](auto it) {
    return with_type(out_dtype, [&](auto ot) {
      return fwd_typed<decltype(it), decltype(ot)>(x0, emb, B, F, D, out, out_stride, false, stream);
    });
  });
}

el_status launch_cat_bwd(const void* dout, el_dtype dout_dtype, int B, int F, int D, int out_stride,
                         void* dx0, void* demb, el_dtype grad_dtype, hipStream_t stream) {
  return with_type(dout_dtype, [&](auto dt) {
    return with_type(grad_dtype, [&](auto gt) {
      return bwd_typed<decltype(dt), decltype(gt)>(dout, B, F, D, out_stride, dx0, demb, stream);
    });
  });
}

el_status launch_emb_cat_fwd(const el_tables& tab, const el_bags& bags, uint32_t flags,
                             const void* x0, el_dtype act_dtype, void* out, int out_stride,
                             hipStream_t stream) {
  const int B = bags.batch, F = tab.num_tables, D = tab.dim;
  const int64_t es = static_cast<int64_t>(dtype_size(act_dtype));
  if ((D * es) % 16 != 0 || (out_stride * es) % 16 != 0)
    return set_error(EL_ERR_UNSUPPORTED, "emb_cat_fwd: D and out_stride must be multiples of 16 bytes of the activation type");
  // x0 block and padding of every row, then the pooled vectors into their blocks
  const el_status st = with_type(act_dtype, [&](auto at) {
    using AT = decltype(at);
    return fwd_typed<AT, AT>(x0, nullptr, B, F, D, out, out_stride, true, stream);
  });
  if (st != EL_OK) return st;
  return launch_emb_bag_fwd(tab, bags, flags, out, act_dtype, stream, 0, B, out_stride, D);
}

}  // namespace el
