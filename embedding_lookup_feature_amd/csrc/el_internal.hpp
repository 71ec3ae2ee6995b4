// el_internal.hpp -- device helpers and kernel launchers shared by the HIP sources of
// libembcore (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <string>

#include "embcore.h"

namespace el {

// ---------------------------------------------------------------------------------------
// Storage formats.  16-bit floats travel as raw uint16_t bit patterns; arithmetic is fp32.
// Conversions to 16-bit round to nearest even (gfx950 v_cvt_pk_bf16_f32 / v_cvt_f16_f32
// under the default round-to-nearest-even mode; denormals kept).
// ---------------------------------------------------------------------------------------
struct F32T {
  using S = float;
  static constexpr el_dtype code = EL_F32;
  __device__ static inline float to_f(S v) { return v; }
  __device__ static inline S from_f(float f) { return f; }
};
struct BF16T {
  using S = uint16_t;
  static constexpr el_dtype code = EL_BF16;
  __device__ static inline float to_f(S v) { return __uint_as_float(static_cast<uint32_t>(v) << 16); }
  __device__ static inline S from_f(float f) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f)); }
};
struct F16T {
  using S = uint16_t;
  static constexpr el_dtype code = EL_F16;
  __device__ static inline float to_f(S v) { return static_cast<float>(__builtin_bit_cast(_Float16, v)); }
  __device__ static inline S from_f(float f) { return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f)); }
};

// Elements of T in one 16-byte vector.
template <class T>
constexpr int epv() { return 16 / static_cast<int>(sizeof(typename T::S)); }

// Unpack a 16-byte vector of T into epv<T>() floats.
template <class T>
__device__ inline void unpack16(const uint4& v, float* f) {
  if constexpr (sizeof(typename T::S) == 4) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  } else {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = T::to_f(static_cast<uint16_t>(w[i] & 0xffffu));
      f[2 * i + 1] = T::to_f(static_cast<uint16_t>(w[i] >> 16));
    }
  }
}

// Store N floats (N = 4 or 8) as T at dst (N * sizeof(T::S) bytes, naturally aligned).
template <class T, int N>
__device__ inline void store_n(typename T::S* dst, const float* f) {
  if constexpr (sizeof(typename T::S) == 4) {
#pragma unroll
    for (int i = 0; i < N; i += 4) {
      uint4 v = {__float_as_uint(f[i]), __float_as_uint(f[i + 1]), __float_as_uint(f[i + 2]),
                 __float_as_uint(f[i + 3])};
      *reinterpret_cast<uint4*>(dst + i) = v;
    }
  } else {
    uint32_t w[N / 2];
#pragma unroll
    for (int i = 0; i < N / 2; ++i)
      w[i] = static_cast<uint32_t>(T::from_f(f[2 * i])) | (static_cast<uint32_t>(T::from_f(f[2 * i + 1])) << 16);
    if constexpr (N == 8) {
      *reinterpret_cast<uint4*>(dst) = uint4{w[0], w[1], w[2], w[3]};
    } else {
      *reinterpret_cast<uint2*>(dst) = uint2{w[0], w[1]};
    }
  }
}

template <class T>
__device__ inline uint4 load16(const typename T::S* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// Streaming (non-temporal) 32-bit load for index / offset streams read once.
__device__ inline int32_t ld_stream(const int32_t* p) { return __builtin_nontemporal_load(p); }
__device__ inline uint32_t ld_stream(const uint32_t* p) { return __builtin_nontemporal_load(p); }

// The hardware hands consecutive workgroups to the 8 XCDs in turn.  This remaps the
// launch order so that each XCD walks one contiguous range of logical blocks (neighbouring
// bags of one table then share that XCD's L2).  `nblocks` must be a multiple of 8.
__device__ inline int xcd_remap(int bid, int nblocks) {
  const int per = nblocks >> 3;
  return (bid & 7) * per + (bid >> 3);
}

inline int round_up8(long long x) { return static_cast<int>((x + 7) / 8 * 8); }

// Floor modulo of a table-local index (--hash_indices): result in [0, n).
__device__ inline int32_t floor_mod(int32_t a, int32_t n) {
  int32_t r = a % n;
  return r < 0 ? r + n : r;
}

// ---------------------------------------------------------------------------------------
// Host side: error text and launch checking.
// ---------------------------------------------------------------------------------------
el_status set_error(el_status st, const std::string& msg);
el_status check_launch(const char* what);

inline size_t dtype_size(el_dtype d) { return d == EL_F32 ? 4 : 2; }
inline bool dtype_valid(int d) { return d == EL_F32 || d == EL_F16 || d == EL_BF16; }

// ---------------------------------------------------------------------------------------
// Launchers (validated arguments only).
// ---------------------------------------------------------------------------------------
// Samples [b0, b0 + Bc) only (Bc < 0: all B).  Pooled vector (b, t) goes to element
// b * ostride + ocol + t * D of `out` (ostride < 0: the [B][F][D] array, F * D, ocol 0).
el_status launch_emb_bag_fwd(const el_tables& tab, const el_bags& bags, uint32_t flags,
                             void* out, el_dtype out_dtype, hipStream_t stream, int b0 = 0,
                             int Bc = -1, int64_t ostride = -1, int ocol = 0);

el_status launch_dot_fwd(const void* x0, const void* emb, el_dtype in_dtype, int B, int F, int D,
                         void* out, el_dtype out_dtype, int out_stride, hipStream_t stream);

el_status launch_dot_bwd(const void* x0, const void* emb, el_dtype in_dtype, int B, int F, int D,
                         const void* dout, el_dtype dout_dtype, int out_stride, void* dx0,
                         void* demb, el_dtype grad_dtype, hipStream_t stream);

// The interaction backward with the pooled vectors rebuilt from the tables (fused gather);
// dout has the activation type.
el_status launch_emb_dot_bwd(const el_tables& tab, const el_bags& bags, uint32_t flags,
                             const void* x0, el_dtype act_dtype, const void* dout, int out_stride,
                             void* dx0, void* demb, el_dtype grad_dtype, hipStream_t stream);

// One tile of the gradient sort: `count` (<= kSortTile) lookups of table t from position
// `start`; the table's lookups start at `seg_start` and own the tiles [first, end).  A tile
// past the last one has count 0.
struct SortTile {
  int32_t t, start, count, seg_start, first, end, pad0, pad1;
};

// Workspace of the gradient path; all pointers 256-byte aligned inside one allocation.
struct GradWorkspace {
  int64_t n = 0;        // lookups
  int passes = 0;       // radix passes
  int rbits = 0;        // digit width of every pass
  int64_t nblocks = 0;  // radix tiles (an upper bound: ceil(n / tile) + tables)
  int64_t nranges = 0;  // reduce ranges (an upper bound: ranges of the fewest lookups)
  size_t bytes = 0;
  uint32_t *keys0 = nullptr, *vals0 = nullptr, *keys1 = nullptr, *vals1 = nullptr;
  int32_t* tile_prefix = nullptr;  // [F+1] tiles of the tables before t
  SortTile* tiles = nullptr;       // [nblocks]
  uint32_t *hist = nullptr, *hist_scan = nullptr;  // digit-major tile counts, scanned per digit
  uint32_t* dtotal = nullptr;                       // per digit: keys with that digit
  uint32_t *flags = nullptr, *flags_scan = nullptr;
  uint32_t* scan_level[4][2] = {};  // per scan level: tile sums, scanned tile sums
  // per reduce range (the sorted lookups one workgroup reduces): fp32 partial row of the run
  // that continues from the previous range (or of the whole range if one run covers it) and
  // of the run that continues into the next range, and flags (bit 0: one run covers the
  // range; bit 1: the range's last run continues into the next range)
  float *range_head = nullptr, *range_tail = nullptr;
  uint32_t* range_flags = nullptr;
};

constexpr int kRadixBits = 9;  // widest radix digit (wider digits measured slower)
static_assert(kRadixBits <= 9, "the sort's histogram and scatter kernels take digits of at most 9 bits");
constexpr int kSortTile = 4096;  // keys per radix tile: 4 waves x 16 steps x 64 lanes
constexpr int kScanTile = 4096;  // elements per scan tile: 256 threads x 16
constexpr int kChunk = 16;         // lookups per lane group in the reduce
constexpr int kMinRange = 4 * kChunk;  // fewest lookups per reduce range (four lane groups)

// Lay out the workspace for n lookups into `tab` in `base` (nullptr: only compute the size).
GradWorkspace plan_grad_workspace(const el_tables& tab, int64_t n, void* base);

// Build keys, radix-sort them; returns the buffers holding the sorted keys / bag ids.
el_status launch_grad_sort_core(const el_tables& tab, const el_bags& bags, uint32_t flags,
                                GradWorkspace& ws, uint32_t** sorted_keys, uint32_t** sorted_vals,
                                hipStream_t stream);

// Where launch_grad_sort_core leaves the sorted keys / bag ids.
void sorted_buffers(const GradWorkspace& ws, uint32_t** sorted_keys, uint32_t** sorted_vals);

el_status launch_segments(const GradWorkspace& ws, const uint32_t* sorted_keys,
                          uint32_t* unique_rows, uint32_t* seg_offsets, uint32_t* num_unique,
                          hipStream_t stream);

el_status launch_reduce_update(const el_tables& tab, const el_bags& bags, const GradWorkspace& ws,
                               const uint32_t* sorted_keys, const uint32_t* sorted_vals,
                               const void* demb, el_dtype grad_dtype, float lr, hipStream_t stream);

el_status launch_exclusive_scan(const uint32_t* in, uint32_t* out, int64_t n,
                                uint32_t* const level[4][2], hipStream_t stream);

// Grid for workgroups of `block` threads that loop over B samples: as many as can be
// resident at once (occupancy from the kernel's registers and `lds_bytes` of LDS), at most B.
int resident_grid(const void* kernel, int B, size_t lds_bytes, int block);

el_status launch_emb_dot_fwd(const el_tables& tab, const el_bags& bags, uint32_t flags,
                             const void* x0, el_dtype act_dtype, void* emb_out, void* out,
                             int out_stride, hipStream_t stream);

// The cat interaction (vectors side by side) and its fused form with the gather.
el_status launch_cat_fwd(const void* x0, const void* emb, el_dtype in_dtype, int B, int F, int D,
                         void* out, el_dtype out_dtype, int out_stride, hipStream_t stream);
el_status launch_cat_bwd(const void* dout, el_dtype dout_dtype, int B, int F, int D, int out_stride,
                         void* dx0, void* demb, el_dtype grad_dtype, hipStream_t stream);
el_status launch_emb_cat_fwd(const el_tables& tab, const el_bags& bags, uint32_t flags,
                             const void* x0, el_dtype act_dtype, void* out, int out_stride,
                             hipStream_t stream);

el_status launch_hbm_calib(int mode, const void* src, void* dst, size_t bytes, const int32_t* idx,
                           int64_t nrows, int row_bytes, hipStream_t stream);

el_status launch_validate(const el_tables& tab, const el_bags& bags, uint32_t flags,
                          int64_t* bad_count, hipStream_t stream);

}  // namespace el
