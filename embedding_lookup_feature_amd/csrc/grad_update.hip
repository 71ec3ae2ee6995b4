// grad_update.hip -- segment reduce of the sorted embedding gradients and the SGD row
// update (gfx950).
//
// Plain SGD on the embedding rows (page "DLRM For PyTorch", §Command-line options --lr):
// W[r] <- W[r] - lr * (sum of the gradients of all lookups of row r).  The lookups arrive
// sorted by row (grad_sort.hip), so the contributions to one row form a run ("segment").
//
// Skewed (Zipf) indices make some segments thousands of lookups long, so the sorted array
// is cut into fixed chunks of 64 lookups instead of one worker per segment:
//   k_seg_chunk : one lane group per chunk sums its runs in order (fp32).  A run that lies
//                 inside the chunk updates its row at once.  The run that continues from
//                 the previous chunk is stored as the chunk's head partial; the run that
//                 continues into the next chunk as its tail partial (the chunk "owns" it);
//                 a chunk that is one run from edge to edge is marked "through".
//   k_seg_fixup : one wavefront per owning chunk finds where its run ends (first chunk
//                 after it that is not "through"), adds tail + head partials in a fixed
//                 order and updates the row.
// Every sum has a fixed association, so results are bitwise reproducible; nothing uses
// atomics and every row is written by exactly one lane group.
#include "el_internal.hpp"

namespace el {
namespace {

// Load N elements of T as floats (N*sizeof(T::S) bytes, naturally aligned).
template <class T, int N>
__device__ inline void load_n(const typename T::S* p, float* f) {
  if constexpr (sizeof(typename T::S) == 4) {
#pragma unroll
    for (int i = 0; i < N; i += 4) unpack16<T>(*reinterpret_cast<const uint4*>(p + i), f + i);
  } else if constexpr (N == 8) {
    unpack16<T>(*reinterpret_cast<const uint4*>(p), f);
  } else {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    f[0] = T::to_f(static_cast<uint16_t>(v.x & 0xffffu));
    f[1] = T::to_f(static_cast<uint16_t>(v.x >> 16));
    f[2] = T::to_f(static_cast<uint16_t>(v.y & 0xffffu));
    f[3] = T::to_f(static_cast<uint16_t>(v.y >> 16));
  }
}

// W[i] <- round(W[i] - lr * g[i]) for the N elements at w (fp32 FMA, one rounding).
template <class WT, int N>
__device__ inline void sgd_n(typename WT::S* w, const float* g, float lr) {
  float cur[N];
  load_n<WT, N>(w, cur);
#pragma unroll
  for (int i = 0; i < N; ++i) cur[i] = fmaf(-lr, g[i], cur[i]);
  store_n<WT, N>(w, cur);
}

template <class GT, class WT, int L, int NVL>
__global__ __launch_bounds__(256) void k_seg_chunk(
    const uint32_t* __restrict__ keys, const uint32_t* __restrict__ vals, int64_t n, int64_t nchunks,
    const typename GT::S* __restrict__ demb, int32_t B, int32_t F, int32_t D, int32_t nvec,
    typename WT::S* __restrict__ W, float lr, float* __restrict__ head, float* __restrict__ tail,
    uint32_t* __restrict__ through, uint32_t* __restrict__ owner) {
  constexpr int E = epv<GT>();
  constexpr uint32_t NONE = 0xffffffffu;  // not a row: rows are < total_rows < 2^32
  const int gl = threadIdx.x % L;
  const int64_t c = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) / L;
  if (c >= nchunks) return;
  const int64_t s = c * kChunk;
  const int64_t e = s + kChunk < n ? s + kChunk : n;
  const uint32_t prev_key = s > 0 ? keys[s - 1] : NONE;
  const uint32_t next_key = e < n ? keys[e] : NONE;

  float acc[NVL][E];
#pragma unroll
  for (int m = 0; m < NVL; ++m)
#pragma unroll
    for (int x = 0; x < E; ++x) acc[m][x] = 0.0f;
  bool first_run = true;
  uint32_t tflag = 0, oflag = 0;

  for (int64_t q0 = s; q0 < e; q0 += 4) {
    uint32_t kq[5];
    uint4 rv[4][NVL];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t q = q0 + u;
      kq[u] = NONE;
      if (q < e) {
        kq[u] = keys[q];
        const uint32_t g = vals[q];
        const uint32_t t = g / static_cast<uint32_t>(B);
        const uint32_t b = g - t * static_cast<uint32_t>(B);
        const typename GT::S* row = demb + (static_cast<int64_t>(b) * F + t) * D;
#pragma unroll
        for (int m = 0; m < NVL; ++m) {
          const int cc = gl + m * L;
          rv[u][m] = cc < nvec ? load16<GT>(row + cc * E) : uint4{0, 0, 0, 0};
        }
      }
    }
    kq[4] = q0 + 4 < e ? keys[q0 + 4] : NONE;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t q = q0 + u;
      if (q >= e) break;
#pragma unroll
      for (int m = 0; m < NVL; ++m) {
        float f[E];
        unpack16<GT>(rv[u][m], f);
#pragma unroll
        for (int x = 0; x < E; ++x) acc[m][x] += f[x];
      }
      const bool last_of_chunk = q + 1 == e;
      if (last_of_chunk || kq[u + 1] != kq[u]) {  // end of a run inside this chunk
        const bool before = first_run && kq[u] == prev_key;
        const bool after = last_of_chunk && kq[u] == next_key;
        if (!before && !after) {
          typename WT::S* wrow = W + static_cast<int64_t>(kq[u]) * D;
#pragma unroll
          for (int m = 0; m < NVL; ++m) {
            const int cc = gl + m * L;
            if (cc < nvec) sgd_n<WT, E>(wrow + cc * E, acc[m], lr);
          }
        } else {
          float* dst = (before ? head : tail) + c * D;
#pragma unroll
          for (int m = 0; m < NVL; ++m) {
            const int cc = gl + m * L;
            if (cc < nvec) store_n<F32T, E>(dst + cc * E, acc[m]);
          }
          if (before && after) tflag = 1;
          if (!before) oflag = 1;
        }
#pragma unroll
        for (int m = 0; m < NVL; ++m)
#pragma unroll
          for (int x = 0; x < E; ++x) acc[m][x] = 0.0f;
        first_run = false;
      }
    }
  }
  if (gl == 0) {
    through[c] = tflag;
    owner[c] = oflag;
  }
}

// One wavefront per chunk; LF lanes cover one fp32 partial row (4 floats per lane and
// vector), NVL vectors per lane.  The NG = 64/LF lane groups sum interleaved chunks; the
// group sums are then added in group order by group 0.
template <class WT, int LF, int NVL>
__global__ __launch_bounds__(256) void k_seg_fixup(
    const uint32_t* __restrict__ keys, int64_t n, int64_t nchunks, int32_t D, int32_t nvec,
    typename WT::S* __restrict__ W, float lr, const float* __restrict__ head,
    const float* __restrict__ tail, const uint32_t* __restrict__ through,
    const uint32_t* __restrict__ owner) {
  constexpr int NG = 64 / LF;
  const int lane = threadIdx.x & 63;
  const int grp = lane / LF, gl = lane % LF;
  const int64_t c = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (c >= nchunks || owner[c] == 0) return;  // wave-uniform
  const int64_t last = (c + 1) * kChunk < n ? (c + 1) * kChunk : n;
  const uint32_t key = keys[last - 1];

  // the run ends in the first chunk after c that is not "through"
  int64_t cend = nchunks - 1;
  for (int64_t b0 = c + 1; b0 < nchunks; b0 += 64) {
    const int64_t cc = b0 + lane;
    const uint64_t m = __ballot(cc < nchunks && through[cc] == 0);
    if (m) {
      cend = b0 + __ffsll(static_cast<unsigned long long>(m)) - 1;
      break;
    }
  }

  float acc[NVL][4];
#pragma unroll
  for (int m = 0; m < NVL; ++m)
#pragma unroll
    for (int x = 0; x < 4; ++x) acc[m][x] = 0.0f;
  for (int64_t cc = c + 1 + grp; cc <= cend; cc += NG) {
    const float* src = head + cc * D;
#pragma unroll
    for (int m = 0; m < NVL; ++m) {
      const int v = gl + m * LF;
      if (v < nvec) {
        float f[4];
        unpack16<F32T>(*reinterpret_cast<const uint4*>(src + v * 4), f);
#pragma unroll
        for (int x = 0; x < 4; ++x) acc[m][x] += f[x];
      }
    }
  }
  // total = tail[c] + group 0 + group 1 + ... (fixed order)
  float tot[NVL][4];
#pragma unroll
  for (int m = 0; m < NVL; ++m) {
    const int v = gl + m * LF;
    if (v < nvec) {
      unpack16<F32T>(*reinterpret_cast<const uint4*>(tail + c * D + v * 4), tot[m]);
    } else {
#pragma unroll
      for (int x = 0; x < 4; ++x) tot[m][x] = 0.0f;
    }
  }
#pragma unroll
  for (int g = 0; g < NG; ++g) {
#pragma unroll
    for (int m = 0; m < NVL; ++m)
#pragma unroll
      for (int x = 0; x < 4; ++x) tot[m][x] += __shfl(acc[m][x], g * LF + gl);
  }
  if (grp == 0) {
    typename WT::S* wrow = W + static_cast<int64_t>(key) * D;
#pragma unroll
    for (int m = 0; m < NVL; ++m) {
      const int v = gl + m * LF;
      if (v < nvec) sgd_n<WT, 4>(wrow + v * 4, tot[m], lr);
    }
  }
}

int blocks_for(int64_t n, int per) { return static_cast<int>((n + per - 1) / per); }

template <class GT, class WT, int L, int NVL>
el_status chunk_t(const el_tables& tab, const el_bags& bags, const GradWorkspace& ws,
                  const uint32_t* keys, const uint32_t* vals, const void* demb, float lr, int nvec,
                  hipStream_t stream) {
  hipLaunchKernelGGL((k_seg_chunk<GT, WT, L, NVL>), dim3(blocks_for(ws.nchunks * L, 256)), dim3(256),
                     0, stream, keys, vals, ws.n, ws.nchunks, static_cast<const typename GT::S*>(demb),
                     bags.batch, tab.num_tables, tab.dim, nvec, static_cast<typename WT::S*>(tab.base),
                     lr, ws.head, ws.tail, ws.through, ws.owner);
  return check_launch("segment_reduce");
}

template <class WT, int LF, int NVL>
el_status fixup_t(const el_tables& tab, const GradWorkspace& ws, const uint32_t* keys, float lr,
                  int nvec, hipStream_t stream) {
  hipLaunchKernelGGL((k_seg_fixup<WT, LF, NVL>), dim3(blocks_for(ws.nchunks, 4)), dim3(256), 0, stream,
                     keys, ws.n, ws.nchunks, tab.dim, nvec, static_cast<typename WT::S*>(tab.base), lr,
                     static_cast<const float*>(ws.head), static_cast<const float*>(ws.tail),
                     static_cast<const uint32_t*>(ws.through), static_cast<const uint32_t*>(ws.owner));
  return check_launch("segment_fixup");
}

template <class GT, class WT>
el_status reduce_typed(const el_tables& tab, const el_bags& bags, const GradWorkspace& ws,
                       const uint32_t* keys, const uint32_t* vals, const void* demb, float lr,
                       hipStream_t stream) {
  const int nvec = static_cast<int>(tab.dim * sizeof(typename GT::S) / 16);
  el_status st;
  if (nvec <= 1) st = chunk_t<GT, WT, 1, 1>(tab, bags, ws, keys, vals, demb, lr, nvec, stream);
  else if (nvec <= 2) st = chunk_t<GT, WT, 2, 1>(tab, bags, ws, keys, vals, demb, lr, nvec, stream);
  else if (nvec <= 4) st = chunk_t<GT, WT, 4, 1>(tab, bags, ws, keys, vals, demb, lr, nvec, stream);
  else if (nvec <= 8) st = chunk_t<GT, WT, 8, 1>(tab, bags, ws, keys, vals, demb, lr, nvec, stream);
  else if (nvec <= 16) st = chunk_t<GT, WT, 16, 1>(tab, bags, ws, keys, vals, demb, lr, nvec, stream);
  else if (nvec <= 32) st = chunk_t<GT, WT, 32, 1>(tab, bags, ws, keys, vals, demb, lr, nvec, stream);
  else if (nvec <= 64) st = chunk_t<GT, WT, 64, 1>(tab, bags, ws, keys, vals, demb, lr, nvec, stream);
  else if (nvec <= 128) st = chunk_t<GT, WT, 64, 2>(tab, bags, ws, keys, vals, demb, lr, nvec, stream);
  else if (nvec <= 256) st = chunk_t<GT, WT, 64, 4>(tab, bags, ws, keys, vals, demb, lr, nvec, stream);
  else return set_error(EL_ERR_UNSUPPORTED, "emb_grad_reduce_update: gradient rows longer than 4096 bytes");
  if (st != EL_OK) return st;
  const int nvf = tab.dim / 4;  // fp32 partial rows: 4 floats per 16-byte vector
  if (nvf <= 1) return fixup_t<WT, 1, 1>(tab, ws, keys, lr, nvf, stream);
  if (nvf <= 2) return fixup_t<WT, 2, 1>(tab, ws, keys, lr, nvf, stream);
  if (nvf <= 4) return fixup_t<WT, 4, 1>(tab, ws, keys, lr, nvf, stream);
  if (nvf <= 8) return fixup_t<WT, 8, 1>(tab, ws, keys, lr, nvf, stream);
  if (nvf <= 16) return fixup_t<WT, 16, 1>(tab, ws, keys, lr, nvf, stream);
  if (nvf <= 32) return fixup_t<WT, 32, 1>(tab, ws, keys, lr, nvf, stream);
  if (nvf <= 64) return fixup_t<WT, 64, 1>(tab, ws, keys, lr, nvf, stream);
  if (nvf <= 128) return fixup_t<WT, 64, 2>(tab, ws, keys, lr, nvf, stream);
  if (nvf <= 256) return fixup_t<WT, 64, 4>(tab, ws, keys, lr, nvf, stream);
  return set_error(EL_ERR_UNSUPPORTED, "emb_grad_reduce_update: dim too large");
}

template <class GT>
el_status reduce_w(const el_tables& tab, const el_bags& bags, const GradWorkspace& ws,
                   const uint32_t* keys, const uint32_t* vals, const void* demb, float lr,
                   hipStream_t stream) {
  switch (tab.dtype) {
    case EL_F32: return reduce_typed<GT, F32T>(tab, bags, ws, keys, vals, demb, lr, stream);
    case EL_F16: return reduce_typed<GT, F16T>(tab, bags, ws, keys, vals, demb, lr, stream);
    case EL_BF16: return reduce_typed<GT, BF16T>(tab, bags, ws, keys, vals, demb, lr, stream);
  }
  return set_error(EL_ERR_INVALID_ARG, "unknown table dtype");
}

}  // namespace

el_status launch_reduce_update(const el_tables& tab, const el_bags& bags, const GradWorkspace& ws,
                               const uint32_t* sorted_keys, const uint32_t* sorted_vals,
                               const void* demb, el_dtype grad_dtype, float lr, hipStream_t stream) {
  switch (grad_dtype) {
    case EL_F32: return reduce_w<F32T>(tab, bags, ws, sorted_keys, sorted_vals, demb, lr, stream);
    case EL_F16: return reduce_w<F16T>(tab, bags, ws, sorted_keys, sorted_vals, demb, lr, stream);
    case EL_BF16: return reduce_w<BF16T>(tab, bags, ws, sorted_keys, sorted_vals, demb, lr, stream);
  }
  return set_error(EL_ERR_INVALID_ARG, "unknown gradient dtype");
}

}  // namespace el
