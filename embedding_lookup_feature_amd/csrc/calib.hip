// calib.hip -- HBM calibration kernels: what plain streaming (and random row gathers) reach
// on this GPU, the ceilings the path's kernels are measured against (gfx950).
//
// The pages measure throughput only (samples/s); the bandwidth ceilings here are this
// build's own yardstick for the gather, interaction and update kernels, which are all
// bandwidth-bound.  Every variant moves 16-byte vectors with K loads in flight per thread
// (all issued before any is used); the streaming variants give a workgroup chunks of
// 256 * K contiguous vectors in turn (load k of a thread at k * 256 vectors from the
// chunk's start: every load instruction of a wavefront covers 1 KiB), looping over the
// buffer.  `bytes` is the total traffic (reads + writes):
//   READ          read `bytes` (an xor of what each thread read goes to one 16-byte slot of
//                 dst per thread, so that nothing is optimised away: a negligible write);
//   WRITE         write `bytes`;
//   COPY          read `bytes` / 2 and write them elsewhere;
//   READ3_WRITE1  three read streams and one write stream of `bytes` / 4 each (output vector
//                 i = xor of input vectors i, i + m and i + 2m, m output vectors): the
//                 read-heavy mix of the gather and the update;
//   GATHER        read whole rows of `row_bytes` at the positions idx[i] of a table at src
//                 (as a hotness-1 embedding gather does) and write each row's first
//                 `bytes` (the whole row if 0; half of it is the mix of fp32 rows pooled
//                 into 16-bit outputs) contiguously to dst: the rows one lane group covers
//                 with 16-byte loads, K rows per group in flight;
//   GATHER_READ   the same rows, only read (an xor per thread to dst).
// The cache policy is the caller's: EL_CALIB_NT_LOADS makes the data loads non-temporal,
// EL_CALIB_NT_STORES the stores; which one is faster depends on the mix (non-temporal loads
// raise a pure streaming read by about a seventh here, and slow a gather that also writes),
// so a ceiling is the best of the policies.
#include "el_internal.hpp"

namespace el {
namespace {

constexpr int K = 8;  // 16-byte vectors in flight per thread

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ inline v4u ld16(const v4u* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}
template <bool NT>
__device__ inline void st16(v4u* p, v4u v) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

template <int MODE, bool NTL, bool NTS>
__global__ __launch_bounds__(256) void k_copy_calib(const v4u* __restrict__ src, v4u* __restrict__ dst,
                                                    int64_t n, v4u* __restrict__ sink) {
  // n: 16-byte vectors per stream
  constexpr int64_t chunk = 256 * K;
  v4u acc = {0u, 0u, 0u, 0u};
  for (int64_t c = blockIdx.x; c * chunk < n; c += gridDim.x) {
    const int64_t base = c * chunk + threadIdx.x;
    if constexpr (MODE == EL_CALIB_WRITE) {
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int64_t i = base + k * 256;
        if (i < n) st16<NTS>(dst + i, v4u{static_cast<uint32_t>(i), 1u, 2u, 3u});
      }
    } else if constexpr (MODE == EL_CALIB_READ3_WRITE1) {
      // output vector i is the xor of input vectors i, i + n and i + 2n: three read streams
      // and one write stream
      v4u a[K], b[K], d[K];
#pragma unroll
      for (int k = 0; k < K; ++k) {
        int64_t i = base + k * 256;
        i = i < n ? i : n - 1;
        a[k] = ld16<NTL>(src + i);
        b[k] = ld16<NTL>(src + n + i);
        d[k] = ld16<NTL>(src + 2 * n + i);
      }
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int64_t i = base + k * 256;
        if (i < n) st16<NTS>(dst + i, a[k] ^ b[k] ^ d[k]);
      }
    } else {
      v4u v[K];
#pragma unroll
      for (int k = 0; k < K; ++k) {
        int64_t i = base + k * 256;
        i = i < n ? i : n - 1;
        v[k] = ld16<NTL>(src + i);
      }
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int64_t i = base + k * 256;
        if constexpr (MODE == EL_CALIB_COPY) {
          if (i < n) st16<NTS>(dst + i, v[k]);
        } else {
          if (i < n) acc ^= v[k];  // clamped re-reads past the end not counted
        }
      }
    }
  }
  if constexpr (MODE == EL_CALIB_READ) sink[static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x] = acc;
}

// Random rows: lane group of L lanes per row (row_vecs 16-byte vectors, up to L per lane
// pass), K rows in flight per group.  WRITE_ROWS: each row is written to dst in order;
// otherwise the rows are only read (an xor per thread goes to dst[thread]).
template <bool WRITE_ROWS, bool NTL, bool NTS>
__global__ __launch_bounds__(256) void k_gather_calib(const v4u* __restrict__ table, int row_vecs,
                                                      const int32_t* __restrict__ idx, int64_t nrows,
                                                      v4u* __restrict__ dst, int L, int out_vecs) {
  const int lane = threadIdx.x & 63;
  const int gl = lane % L;
  const int64_t groups = static_cast<int64_t>(gridDim.x) * (256 / L);
  const int64_t g = static_cast<int64_t>(blockIdx.x) * (256 / L) + threadIdx.x / L;
  v4u acc = {0u, 0u, 0u, 0u};
  for (int64_t r0 = g; r0 < nrows; r0 += groups * K) {
    v4u v[K];
    int64_t rr[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      int64_t r = r0 + static_cast<int64_t>(k) * groups;
      rr[k] = r;
      r = r < nrows ? r : nrows - 1;
      const int64_t row = idx[r];
      v[k] = gl < row_vecs ? ld16<NTL>(table + row * row_vecs + gl) : v4u{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
      if constexpr (WRITE_ROWS) {
        if (rr[k] < nrows && gl < out_vecs) st16<NTS>(dst + rr[k] * out_vecs + gl, v[k]);
      } else {
        if (rr[k] < nrows) acc ^= v[k];  // clamped re-reads past the end not counted
      }
    }
  }
  if constexpr (!WRITE_ROWS) dst[static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x] = acc;
}

template <bool NTL, bool NTS>
el_status launch_policy(int mode, const void* src, void* dst, size_t bytes, const int32_t* idx,
                        int64_t nrows, int row_bytes, hipStream_t stream) {
  const int grid = 256 * 8;  // 8 workgroups of 256 threads per CU, looping over the buffer
  if (mode == EL_CALIB_GATHER || mode == EL_CALIB_GATHER_READ) {
    const int row_vecs = row_bytes / 16;
    int L = 1;
    while (L < row_vecs && L < 64) L <<= 1;
    // GATHER: `bytes` = bytes written per row (the row's first part; 0: the whole row)
    const int out_vecs = bytes ? static_cast<int>(bytes / 16) : row_vecs;
    if (mode == EL_CALIB_GATHER)
      hipLaunchKernelGGL((k_gather_calib<true, NTL, NTS>), dim3(grid), dim3(256), 0, stream,
                         static_cast<const v4u*>(src), row_vecs, idx, nrows, static_cast<v4u*>(dst), L,
                         out_vecs);
    else
      hipLaunchKernelGGL((k_gather_calib<false, NTL, NTS>), dim3(grid), dim3(256), 0, stream,
                         static_cast<const v4u*>(src), row_vecs, idx, nrows, static_cast<v4u*>(dst), L,
                         out_vecs);
    return check_launch("el_hbm_calib");
  }
  const int64_t vecs = static_cast<int64_t>(bytes / 16);
  const v4u* s = static_cast<const v4u*>(src);
  v4u* d = static_cast<v4u*>(dst);
  switch (mode) {
    case EL_CALIB_READ:
      hipLaunchKernelGGL((k_copy_calib<EL_CALIB_READ, NTL, NTS>), dim3(grid), dim3(256), 0, stream, s, d, vecs, d);
      break;
    case EL_CALIB_WRITE:
      hipLaunchKernelGGL((k_copy_calib<EL_CALIB_WRITE, NTL, NTS>), dim3(grid), dim3(256), 0, stream, s, d, vecs, d);
      break;
    case EL_CALIB_COPY:
      hipLaunchKernelGGL((k_copy_calib<EL_CALIB_COPY, NTL, NTS>), dim3(grid), dim3(256), 0, stream, s, d,
                         vecs / 2, d);
      break;
    case EL_CALIB_READ3_WRITE1:
      hipLaunchKernelGGL((k_copy_calib<EL_CALIB_READ3_WRITE1, NTL, NTS>), dim3(grid), dim3(256), 0, stream, s,
                         d, vecs / 4, d);
      break;
    default:
      return set_error(EL_ERR_INVALID_ARG, "el_hbm_calib: unknown mode");
  }
  return check_launch("el_hbm_calib");
}

}  // namespace

el_status launch_hbm_calib(int mode, const void* src, void* dst, size_t bytes, const int32_t* idx,
                           int64_t nrows, int row_bytes, hipStream_t stream) {
  const bool ntl = (mode & EL_CALIB_NT_LOADS) != 0, nts = (mode & EL_CALIB_NT_STORES) != 0;
  const int base = mode & EL_CALIB_MODE_MASK;
  if (ntl && nts) return launch_policy<true, true>(base, src, dst, bytes, idx, nrows, row_bytes, stream);
  if (ntl) return launch_policy<true, false>(base, src, dst, bytes, idx, nrows, row_bytes, stream);
  if (nts) return launch_policy<false, true>(base, src, dst, bytes, idx, nrows, row_bytes, stream);
  return launch_policy<false, false>(base, src, dst, bytes, idx, nrows, row_bytes, stream);
}

}  // namespace el
