// calib.hip -- HBM calibration kernels: what plain streaming (and random row gathers) reach
// on this GPU, the ceilings the path's kernels are measured against (gfx950).
//
// The pages measure throughput only (samples/s); the bandwidth ceilings here are this
// build's own yardstick for the gather, interaction and update kernels, which are all
// bandwidth-bound.  Every variant moves 16-byte vectors, each thread keeps K loads in flight
// (all issued before any is used), and the grid loops over the buffer; `bytes` is the
// total traffic (reads + writes):
//   READ          read `bytes` (an xor of what each thread read goes to one 16-byte slot of
//                 dst per thread, so that nothing is optimised away: a negligible write);
//   WRITE         write `bytes`;
//   COPY          read `bytes` / 2 and write them elsewhere;
//   READ3_WRITE1  read three quarters of `bytes` and write one quarter (output vector i =
//                 xor of input vectors 3i .. 3i+2): the read-heavy mix of the gather and the
//                 update;
//   GATHER        read whole rows of `row_bytes` at the positions idx[i] of a table at src
//                 (as a hotness-1 embedding gather does) and write each row's first
//                 `bytes` (the whole row if 0; half of it is the mix of fp32 rows pooled
//                 into 16-bit outputs) contiguously to dst: the rows one lane group covers
//                 with 16-byte loads, K rows per group in flight;
//   GATHER_READ   the same rows, only read (an xor per thread to dst).
#include "el_internal.hpp"

namespace el {
namespace {

constexpr int K = 8;  // 16-byte vectors in flight per thread

__device__ inline uint4 xor4(uint4 a, uint4 b) { return uint4{a.x ^ b.x, a.y ^ b.y, a.z ^ b.z, a.w ^ b.w}; }

template <int MODE>
__global__ __launch_bounds__(256) void k_copy_calib(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                    int64_t n, uint4* __restrict__ sink) {
  // n: 16-byte vectors per stream
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t nthreads = static_cast<int64_t>(gridDim.x) * 256;
  uint4 acc = uint4{0u, 0u, 0u, 0u};
  for (int64_t base = tid; base < n; base += nthreads * K) {
    if constexpr (MODE == EL_CALIB_WRITE) {
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int64_t i = base + static_cast<int64_t>(k) * nthreads;
        if (i < n) dst[i] = uint4{static_cast<uint32_t>(i), 1u, 2u, 3u};
      }
    } else if constexpr (MODE == EL_CALIB_READ3_WRITE1) {
      // output vector i is the xor of input vectors 3i, 3i+1, 3i+2: one read stream three
      // times as fast as the write stream
      uint4 a[K], b[K], c[K];
#pragma unroll
      for (int k = 0; k < K; ++k) {
        int64_t i = base + static_cast<int64_t>(k) * nthreads;
        i = i < n ? i : n - 1;
        a[k] = src[3 * i];
        b[k] = src[3 * i + 1];
        c[k] = src[3 * i + 2];
      }
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int64_t i = base + static_cast<int64_t>(k) * nthreads;
        if (i < n) dst[i] = xor4(xor4(a[k], b[k]), c[k]);
      }
    } else {
      uint4 v[K];
#pragma unroll
      for (int k = 0; k < K; ++k) {
        int64_t i = base + static_cast<int64_t>(k) * nthreads;
        i = i < n ? i : n - 1;
        v[k] = src[i];
      }
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int64_t i = base + static_cast<int64_t>(k) * nthreads;
        if constexpr (MODE == EL_CALIB_COPY) {
          if (i < n) dst[i] = v[k];
        } else {
          if (i < n) acc = xor4(acc, v[k]);  // clamped re-reads past the end not counted
        }
      }
    }
  }
  if constexpr (MODE == EL_CALIB_READ) sink[tid] = acc;
}

// Random rows: lane group of L lanes per row (row_vecs 16-byte vectors, up to L per lane
// pass), K rows in flight per group.  WRITE_ROWS: each row is written to dst in order;
// otherwise the rows are only read (an xor per thread goes to dst[thread]).
template <bool WRITE_ROWS>
__global__ __launch_bounds__(256) void k_gather_calib(const uint4* __restrict__ table, int row_vecs,
                                                      const int32_t* __restrict__ idx, int64_t nrows,
                                                      uint4* __restrict__ dst, int L, int out_vecs) {
  const int lane = threadIdx.x & 63;
  const int gl = lane % L;
  const int64_t groups = static_cast<int64_t>(gridDim.x) * (256 / L);
  const int64_t g = static_cast<int64_t>(blockIdx.x) * (256 / L) + threadIdx.x / L;
  uint4 acc = uint4{0u, 0u, 0u, 0u};
  for (int64_t r0 = g; r0 < nrows; r0 += groups * K) {
    uint4 v[K];
    int64_t rr[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      int64_t r = r0 + static_cast<int64_t>(k) * groups;
      rr[k] = r;
      r = r < nrows ? r : nrows - 1;
      const int64_t row = idx[r];
      v[k] = gl < row_vecs ? table[row * row_vecs + gl] : uint4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
      if constexpr (WRITE_ROWS) {
        if (rr[k] < nrows && gl < out_vecs) dst[rr[k] * out_vecs + gl] = v[k];
      } else {
        if (rr[k] < nrows) acc = xor4(acc, v[k]);  // clamped re-reads past the end not counted
      }
    }
  }
  if constexpr (!WRITE_ROWS) dst[static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x] = acc;
}

}  // namespace

el_status launch_hbm_calib(int mode, const void* src, void* dst, size_t bytes, const int32_t* idx,
                           int64_t nrows, int row_bytes, hipStream_t stream) {
  const int grid = 256 * 8;  // 8 workgroups of 256 threads per CU, looping over the buffer
  if (mode == EL_CALIB_GATHER || mode == EL_CALIB_GATHER_READ) {
    const int row_vecs = row_bytes / 16;
    int L = 1;
    while (L < row_vecs && L < 64) L <<= 1;
    // GATHER: `bytes` = bytes written per row (the row's first part; 0: the whole row)
    const int out_vecs = bytes ? static_cast<int>(bytes / 16) : row_vecs;
    if (mode == EL_CALIB_GATHER)
      hipLaunchKernelGGL(k_gather_calib<true>, dim3(grid), dim3(256), 0, stream,
                         static_cast<const uint4*>(src), row_vecs, idx, nrows, static_cast<uint4*>(dst), L,
                         out_vecs);
    else
      hipLaunchKernelGGL(k_gather_calib<false>, dim3(grid), dim3(256), 0, stream,
                         static_cast<const uint4*>(src), row_vecs, idx, nrows, static_cast<uint4*>(dst), L,
                         out_vecs);
    return check_launch("el_hbm_calib");
  }
  const int64_t vecs = static_cast<int64_t>(bytes / 16);
  const uint4* s = static_cast<const uint4*>(src);
  uint4* d = static_cast<uint4*>(dst);
  switch (mode) {
    case EL_CALIB_READ:
      hipLaunchKernelGGL(k_copy_calib<EL_CALIB_READ>, dim3(grid), dim3(256), 0, stream, s, d, vecs, d);
      break;
    case EL_CALIB_WRITE:
      hipLaunchKernelGGL(k_copy_calib<EL_CALIB_WRITE>, dim3(grid), dim3(256), 0, stream, s, d, vecs, d);
      break;
    case EL_CALIB_COPY:
      hipLaunchKernelGGL(k_copy_calib<EL_CALIB_COPY>, dim3(grid), dim3(256), 0, stream, s, d, vecs / 2, d);
      break;
    case EL_CALIB_READ3_WRITE1:
      hipLaunchKernelGGL(k_copy_calib<EL_CALIB_READ3_WRITE1>, dim3(grid), dim3(256), 0, stream, s, d,
                         vecs / 4, d);
      break;
    default:
      return set_error(EL_ERR_INVALID_ARG, "el_hbm_calib: unknown mode");
  }
  return check_launch("el_hbm_calib");
}

}  // namespace el
