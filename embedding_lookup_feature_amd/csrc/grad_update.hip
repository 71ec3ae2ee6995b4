// grad_update.hip -- segment reduce of the sorted embedding gradients and the SGD row
// update (gfx950).
//
// Plain SGD on the embedding rows (page "DLRM For PyTorch", §Command-line options --lr):
// W[r] <- W[r] - lr * (sum of the gradients of all lookups of row r).  The lookups arrive
// sorted by row (grad_sort.hip), so the contributions to one row form a run ("segment").
//
// Skewed (Zipf) indices make some runs thousands of lookups long, so the sorted array is
// cut into fixed chunks of 16 lookups instead of one worker per run:
//   k_seg_chunk : one lane group per chunk.  Every lane covers 4 consecutive elements of a
//                 row.  The group (1) loads the chunk's 16 row numbers and bag ids, (2)
//                 issues all 16 gradient-row loads and the table-row loads of every run that
//                 starts and ends inside the chunk, then (3) sums the runs in order (fp32),
//                 updates those rows and stores the partials of the runs crossing the chunk
//                 edges: the run continuing from the previous chunk is the chunk's head
//                 partial, the run continuing into the next chunk its tail partial (the
//                 chunk "owns" it); a chunk that is one run from edge to edge is "through".
//                 No load is issued after a store, so a group never waits for its stores
//                 (loads and stores share one completion counter on this architecture).
//   k_seg_blocksum : for every block of 64 chunks that one run covers entirely ("through"
//                 chunks only), the sum of their head partials.
//   k_seg_fixup : one wavefront per 64 chunks.  An owning chunk's run ends at the first
//                 chunk after it that is not "through"; runs ending within a few chunks are
//                 finished by small lane groups side by side (tail + head partials in chunk
//                 order), longer ones by the whole wavefront, skipping whole "through"
//                 blocks via their block sums.
// Every sum has a fixed association, so results are bitwise reproducible; nothing uses
// atomics and every row is written by exactly one lane group.
#include <type_traits>

#include "el_internal.hpp"

namespace el {
namespace {

// 4 consecutive elements of T as floats / back (8 or 16 bytes, naturally aligned).
template <class T>
__device__ inline void load4(const typename T::S* p, float* f) {
  if constexpr (sizeof(typename T::S) == 4) {
    unpack16<T>(*reinterpret_cast<const uint4*>(p), f);
  } else {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    f[0] = T::to_f(static_cast<uint16_t>(v.x & 0xffffu));
    f[1] = T::to_f(static_cast<uint16_t>(v.x >> 16));
    f[2] = T::to_f(static_cast<uint16_t>(v.y & 0xffffu));
    f[3] = T::to_f(static_cast<uint16_t>(v.y >> 16));
  }
}

// Raw 4-element load (kept as bits until used, so that issuing it never waits).
template <class T>
struct Raw4 {
  using type = typename std::conditional<sizeof(typename T::S) == 4, uint4, uint2>::type;
};
template <class T>
__device__ inline typename Raw4<T>::type load4_raw(const typename T::S* p) {
  return *reinterpret_cast<const typename Raw4<T>::type*>(p);
}
template <class T>
__device__ inline void unpack4(const typename Raw4<T>::type& v, float* f) {
  if constexpr (sizeof(typename T::S) == 4) {
    unpack16<T>(v, f);
  } else {
    f[0] = T::to_f(static_cast<uint16_t>(v.x & 0xffffu));
    f[1] = T::to_f(static_cast<uint16_t>(v.x >> 16));
    f[2] = T::to_f(static_cast<uint16_t>(v.y & 0xffffu));
    f[3] = T::to_f(static_cast<uint16_t>(v.y >> 16));
  }
}

// W[i] <- round(W[i] - lr * g[i]) for 4 elements at w, from the loaded old values (fp32 FMA,
// one rounding).
template <class WT>
__device__ inline void sgd4(typename WT::S* w, const typename Raw4<WT>::type& old, const float* g,
                            float lr) {
  float cur[4];
  unpack4<WT>(old, cur);
#pragma unroll
  for (int i = 0; i < 4; ++i) cur[i] = fmaf(-lr, g[i], cur[i]);
  store_n<WT, 4>(w, cur);
}

constexpr int CH = kChunk;  // lookups per chunk
constexpr int kFixChunks = 32;  // chunks per fix-up wavefront (owners on lanes 0..31)

// L lanes per row, each covering 4 elements per vector, NV vectors per lane.
template <class GT, class WT, int L, int NV>
__global__ __launch_bounds__(256) void k_seg_chunk(
    const uint32_t* __restrict__ keys, const uint32_t* __restrict__ vals, int64_t n, int64_t nchunks,
    const typename GT::S* __restrict__ demb, int32_t B, int32_t F, int32_t D, int32_t nv4,
    typename WT::S* __restrict__ W, float lr, float* __restrict__ head, float* __restrict__ tail,
    uint32_t* __restrict__ through, uint32_t* __restrict__ owner) {
  static_assert(CH <= 64, "one row number per lane and 16-lane sub-steps");
  constexpr uint32_t NONE = 0xffffffffu;  // not a row: rows are < total_rows < 2^32
  constexpr int KPL = CH > L ? CH / L : 1;  // row numbers per lane
  const int lane = threadIdx.x & 63;
  const int gl = lane % L;
  const int gbase = lane - gl;  // first lane of the group
  const int64_t c = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) / L;
  if (c >= nchunks) return;  // group-uniform
  const int64_t s = c * CH;
  const int cnt = static_cast<int>(n - s < CH ? n - s : CH);  // lookups in this chunk, >= 1

  // (1) row numbers and bag ids of the chunk, and the neighbours across its edges
  uint32_t kr[KPL], vr[KPL];
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    const int q = gl + j * L;
    const int qc = q < cnt ? q : cnt - 1;
    kr[j] = keys[s + qc];
    vr[j] = vals[s + qc];
  }
  const uint32_t prev_key = s > 0 ? keys[s - 1] : NONE;
  const uint32_t next_key = s + cnt < n ? keys[s + cnt] : NONE;

  auto key_at = [&](int q) { return static_cast<uint32_t>(__shfl(static_cast<int>(kr[q / L]), gbase + q % L)); };
  auto val_at = [&](int q) { return static_cast<uint32_t>(__shfl(static_cast<int>(vr[q / L]), gbase + q % L)); };
  const uint32_t k_first = key_at(0);
  const uint32_t k_last = key_at(cnt - 1);  // cnt - 1 is group-uniform
  const bool first_before = k_first == prev_key;  // the first run started in an earlier chunk
  const bool last_after = k_last == next_key;     // the last run continues in a later chunk

  // (2) all loads: gradient rows, and the table rows of runs that lie inside the chunk
  typename Raw4<GT>::type rows[CH][NV];
  typename Raw4<WT>::type wold[CH][NV];
  uint32_t kq[CH];
#pragma unroll
  for (int q = 0; q < CH; ++q) {
    kq[q] = key_at(q < cnt ? q : cnt - 1);
    const uint32_t g = val_at(q < cnt ? q : cnt - 1);
    const uint32_t t = g / static_cast<uint32_t>(B);
    const uint32_t b = g - t * static_cast<uint32_t>(B);
    const typename GT::S* row = demb + (static_cast<int64_t>(b) * F + t) * D;
#pragma unroll
    for (int m = 0; m < NV; ++m) {
      const int v = gl + m * L;
      rows[q][m] = load4_raw<GT>(row + (v < nv4 ? v : nv4 - 1) * 4);
    }
  }
#pragma unroll
  for (int q = 0; q < CH; ++q) {
    const bool end = q < cnt && (q == cnt - 1 || kq[q + 1 < CH ? q + 1 : q] != kq[q]);
    const bool inside = end && !(kq[q] == k_first && first_before) && !(kq[q] == k_last && last_after);
    // unconditional, so the compiler can count outstanding loads exactly; positions that
    // do not end an inside run re-read the first run's row (a cached line) and ignore it
    const int64_t wr = inside ? kq[q] : k_first;
#pragma unroll
    for (int m = 0; m < NV; ++m) {
      const int v = gl + m * L;
      wold[q][m] = load4_raw<WT>(W + wr * D + (v < nv4 ? v : nv4 - 1) * 4);
    }
  }

  // (3) run sums in order, row updates and edge partials
  float acc[NV][4];
#pragma unroll
  for (int m = 0; m < NV; ++m)
#pragma unroll
    for (int x = 0; x < 4; ++x) acc[m][x] = 0.0f;
#pragma unroll
  for (int q = 0; q < CH; ++q) {
    if (q < cnt) {
#pragma unroll
      for (int m = 0; m < NV; ++m) {
        float f[4];
        unpack4<GT>(rows[q][m], f);
#pragma unroll
        for (int x = 0; x < 4; ++x) acc[m][x] += f[x];
      }
      const bool end = q == cnt - 1 || kq[q + 1 < CH ? q + 1 : q] != kq[q];
      if (end) {
        const bool before = kq[q] == k_first && first_before;
        const bool after = kq[q] == k_last && last_after;
#pragma unroll
        for (int m = 0; m < NV; ++m) {
          const int v = gl + m * L;
          if (v < nv4) {
            if (!before && !after)
              sgd4<WT>(W + static_cast<int64_t>(kq[q]) * D + v * 4, wold[q][m], acc[m], lr);
            else
              store_n<F32T, 4>((before ? head : tail) + c * D + v * 4, acc[m]);
          }
        }
#pragma unroll
        for (int m = 0; m < NV; ++m)
#pragma unroll
          for (int x = 0; x < 4; ++x) acc[m][x] = 0.0f;
      }
    }
  }
  if (gl == 0) {
    through[c] = (k_first == k_last && first_before && last_after) ? 1u : 0u;
    owner[c] = (last_after && !(k_last == k_first && first_before)) ? 1u : 0u;
  }
}

// Sum of the fp32 rows first..last (inclusive) of a [rows][D] array into acc, for one
// wavefront: NG = 64/LF lane groups take rows first+g, first+g+NG, ... with UF loads in
// flight each, and the group sums are added in group order (returned in every group).
// The association depends only on (first, last), so results are reproducible.
template <int LF, int NV, int UF>
__device__ inline void sum_rows(const float* __restrict__ base, int64_t first, int64_t last, int D,
                                int nv4, float (&acc)[NV][4]) {
  constexpr int NG = 64 / LF;
  const int lane = threadIdx.x & 63;
  const int grp = lane / LF, gl = lane % LF;
  float part[NV][4];
#pragma unroll
  for (int m = 0; m < NV; ++m)
#pragma unroll
    for (int x = 0; x < 4; ++x) part[m][x] = 0.0f;
  for (int64_t c0 = first + grp; c0 <= last; c0 += NG * UF) {
    uint4 p[UF][NV];
#pragma unroll
    for (int u = 0; u < UF; ++u) {
      int64_t cc = c0 + static_cast<int64_t>(u) * NG;
      cc = cc <= last ? cc : last;
#pragma unroll
      for (int m = 0; m < NV; ++m) {
        const int v = gl + m * LF;
        p[u][m] = *reinterpret_cast<const uint4*>(base + cc * D + (v < nv4 ? v : nv4 - 1) * 4);
      }
    }
#pragma unroll
    for (int u = 0; u < UF; ++u) {
      if (c0 + static_cast<int64_t>(u) * NG <= last) {
#pragma unroll
        for (int m = 0; m < NV; ++m) {
          float f[4];
          unpack16<F32T>(p[u][m], f);
#pragma unroll
          for (int x = 0; x < 4; ++x) part[m][x] += f[x];
        }
      }
    }
  }
#pragma unroll
  for (int g = 0; g < NG; ++g) {
#pragma unroll
    for (int m = 0; m < NV; ++m)
#pragma unroll
      for (int x = 0; x < 4; ++x) acc[m][x] += __shfl(part[m][x], g * LF + gl);
  }
}

// One wavefront per block of kBlockChunks chunks: if every chunk of the block is "through"
// (one run covers the whole block), store the sum of their head partials.
template <int LF, int NV>
__global__ __launch_bounds__(256) void k_seg_blocksum(const float* __restrict__ head,
                                                      const uint32_t* __restrict__ through,
                                                      int64_t nchunks, int64_t nblk, int32_t D,
                                                      int32_t nv4, float* __restrict__ bsum,
                                                      uint32_t* __restrict__ bthrough) {
  const int lane = threadIdx.x & 63;
  const int64_t j = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (j >= nblk) return;
  const int64_t c0 = j * kBlockChunks;
  const int64_t cc = c0 + lane;
  const uint64_t m = __ballot(cc < nchunks && through[cc] != 0);
  const bool full = m == ~0ull;
  if (lane == 0) bthrough[j] = full ? 1u : 0u;
  if (!full) return;
  float acc[NV][4];
#pragma unroll
  for (int q = 0; q < NV; ++q)
#pragma unroll
    for (int x = 0; x < 4; ++x) acc[q][x] = 0.0f;
  sum_rows<LF, NV, 16>(head, c0, c0 + kBlockChunks - 1, D, nv4, acc);
  const int gl = lane % LF;
  if (lane < LF) {
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      const int v = gl + q * LF;
      if (v < nv4) store_n<F32T, 4>(bsum + j * D + v * 4, acc[q]);
    }
  }
}

// First index i >= from with flag[i] == 0 (flags past n count as 0); one wavefront.
__device__ inline int64_t first_zero(const uint32_t* __restrict__ flag, int64_t from, int64_t n) {
  const int lane = threadIdx.x & 63;
  for (int64_t b0 = from;; b0 += 64) {
    const int64_t i = b0 + lane;
    const uint64_t m = __ballot(i >= n || flag[i] == 0);
    if (m) return b0 + __ffsll(static_cast<unsigned long long>(m)) - 1;
  }
}

// Row update of a long run owned by chunk c (whole wavefront): total = tail partial + head
// partials of the chunks up to the one where the run ends, taking whole "through" blocks
// from their block sums.
template <class WT, int LF, int NV>
__device__ inline void fix_long(int64_t c, uint32_t key, int64_t nchunks, int32_t D, int32_t nv4,
                                typename WT::S* __restrict__ W, float lr,
                                const float* __restrict__ head, const float* __restrict__ tail,
                                const uint32_t* __restrict__ through, const float* __restrict__ bsum,
                                const uint32_t* __restrict__ bthrough, int64_t nblk) {
  const int lane = threadIdx.x & 63;
  const int gl = lane % LF;
  typename Raw4<WT>::type wold[NV];
#pragma unroll
  for (int m = 0; m < NV; ++m) {
    const int v = gl + m * LF;
    wold[m] = load4_raw<WT>(W + static_cast<int64_t>(key) * D + (v < nv4 ? v : nv4 - 1) * 4);
  }
  float tot[NV][4];
#pragma unroll
  for (int m = 0; m < NV; ++m) {
    const int v = gl + m * LF;
    unpack16<F32T>(*reinterpret_cast<const uint4*>(tail + c * D + (v < nv4 ? v : nv4 - 1) * 4), tot[m]);
  }
  // where does the run end?  first a window of 64 chunks, then whole blocks
  const int64_t cw = first_zero(through, c + 1, c + 65 < nchunks ? c + 65 : nchunks);
  if (cw < c + 65 && cw < nchunks && through[cw] == 0) {
    sum_rows<LF, NV, 16>(head, c + 1, cw, D, nv4, tot);  // ends within the window
  } else {
    // chunks c+1 .. c+64 are all "through"; continue from the next block boundary
    const int64_t jb = (c + 1 + kBlockChunks - 1) / kBlockChunks;  // first block starting after c
    const int64_t cb = jb * kBlockChunks;                           // <= c + 64
    const int64_t je = first_zero(bthrough, jb, nblk);              // first block not fully through
    const int64_t cend = first_zero(through, je * kBlockChunks, nchunks);
    if (cb > c + 1) sum_rows<LF, NV, 16>(head, c + 1, cb - 1, D, nv4, tot);
    if (je > jb) sum_rows<LF, NV, 16>(bsum, jb, je - 1, D, nv4, tot);
    sum_rows<LF, NV, 16>(head, je * kBlockChunks, cend, D, nv4, tot);
  }
  if (lane < LF) {
#pragma unroll
    for (int m = 0; m < NV; ++m) {
      const int v = gl + m * LF;
      if (v < nv4) sgd4<WT>(W + static_cast<int64_t>(key) * D + v * 4, wold[m], tot[m], lr);
    }
  }
}

// One wavefront per kFixChunks (32) consecutive chunks.  Ballots give the "owner" flags of
// its chunks and the "through" flags of the 128 chunks from its first, so every owning chunk
// sees at once where its run ends.  Runs ending at most S chunks after their owner ("short", the common case) are
// finished by lane groups of LG lanes, 64/LG owners side by side: the group loads the tail
// partial, the S head partials (clamped to the end chunk) and the table row together, adds
// them in chunk order and updates the row.  Longer runs are then finished one after the
// other by the whole wavefront (fix_long).
template <class WT, int LG, int NVG, int S, int LF, int NV>
__global__ __launch_bounds__(256) void k_seg_fixup(
    const uint32_t* __restrict__ keys, int64_t n, int64_t nchunks, int32_t D, int32_t nv4,
    typename WT::S* __restrict__ W, float lr, const float* __restrict__ head,
    const float* __restrict__ tail, const uint32_t* __restrict__ through,
    const uint32_t* __restrict__ owner, const float* __restrict__ bsum,
    const uint32_t* __restrict__ bthrough, int64_t nblk) {
  constexpr int NGW = 64 / LG;  // owner groups per wavefront
  const int lane = threadIdx.x & 63;
  const int64_t c0 = (static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6)) * kFixChunks;
  if (c0 >= nchunks) return;  // wave-uniform
  const int64_t cl = c0 + lane, ch = c0 + 64 + lane;
  const bool own = lane < kFixChunks && cl < nchunks && owner[cl] != 0;
  const uint64_t tm0 = __ballot(cl < nchunks && through[cl] != 0);
  const uint64_t tm1 = __ballot(ch < nchunks && through[ch] != 0);
  // row of this lane's chunk (the last key of the chunk: the run it owns)
  const int64_t lastpos = (cl + 1) * CH < n ? (cl + 1) * CH : n;
  const uint32_t keyl = cl < nchunks ? keys[lastpos - 1] : 0u;
  // end chunk (relative to c0) of the run owned by chunk cl: first non-"through" chunk after it
  int e = 128;
  {
    const uint64_t z0 = lane < 63 ? (~tm0 & (~0ull << (lane + 1))) : 0ull;
    if (z0) e = __ffsll(static_cast<unsigned long long>(z0)) - 1;
    else if (~tm1) e = 64 + __ffsll(static_cast<unsigned long long>(~tm1)) - 1;
  }
  const bool is_short = own && e - lane <= S;
  const uint64_t ms = __ballot(is_short);
  uint64_t ml = __ballot(own && !is_short);
  const int ns = __popcll(ms);
  // ranks: short owners first in chunk order, then every other lane (a permutation of lanes)
  const uint64_t lt = (1ull << lane) - 1ull;
  const int rank = is_short ? __popcll(ms & lt) : ns + __popcll(~ms & lt);
  // lane r receives the lane index of the owner of rank r
  const int who = __builtin_amdgcn_ds_permute(rank * 4, lane);
  const int grp = lane / LG, gl = lane % LG;
  for (int r0 = 0; r0 < ns; r0 += NGW) {  // wave-uniform trip count
    const int R = r0 + grp;
    const int i = __shfl(who, R < ns ? R : 0);
    const int ei = __shfl(e, i);
    const uint32_t key = static_cast<uint32_t>(__shfl(static_cast<int>(keyl), i));
    if (R < ns) {  // group-uniform
      const int64_t c = c0 + i, ce = c0 + ei;  // c < ce <= c + S
      typename Raw4<WT>::type wold[NVG];
      uint4 tl[NVG], hd[S][NVG];
#pragma unroll
      for (int m = 0; m < NVG; ++m) {
        const int v = gl + m * LG;
        const int vo = (v < nv4 ? v : nv4 - 1) * 4;
        wold[m] = load4_raw<WT>(W + static_cast<int64_t>(key) * D + vo);
        tl[m] = *reinterpret_cast<const uint4*>(tail + c * D + vo);
#pragma unroll
        for (int j = 0; j < S; ++j) {
          const int64_t cc = c + 1 + j <= ce ? c + 1 + j : ce;
          hd[j][m] = *reinterpret_cast<const uint4*>(head + cc * D + vo);
        }
      }
#pragma unroll
      for (int m = 0; m < NVG; ++m) {
        const int v = gl + m * LG;
        float tot[4], f[4];
        unpack16<F32T>(tl[m], tot);
#pragma unroll
        for (int j = 0; j < S; ++j) {
          if (c + 1 + j <= ce) {
            unpack16<F32T>(hd[j][m], f);
#pragma unroll
            for (int x = 0; x < 4; ++x) tot[x] += f[x];
          }
        }
        if (v < nv4) sgd4<WT>(W + static_cast<int64_t>(key) * D + v * 4, wold[m], tot, lr);
      }
    }
  }
  while (ml) {  // wave-uniform
    const int i = __ffsll(static_cast<unsigned long long>(ml)) - 1;
    ml &= ml - 1;
    const uint32_t key = static_cast<uint32_t>(__shfl(static_cast<int>(keyl), i));
    fix_long<WT, LF, NV>(c0 + i, key, nchunks, D, nv4, W, lr, head, tail, through, bsum, bthrough, nblk);
  }
}

int blocks_for(int64_t n, int per) { return static_cast<int>((n + per - 1) / per); }

template <class GT, class WT, int L, int NV>
el_status chunk_t(const el_tables& tab, const el_bags& bags, const GradWorkspace& ws,
                  const uint32_t* keys, const uint32_t* vals, const void* demb, float lr, int nv4,
                  hipStream_t stream) {
  hipLaunchKernelGGL((k_seg_chunk<GT, WT, L, NV>), dim3(blocks_for(ws.nchunks * L, 256)), dim3(256),
                     0, stream, keys, vals, ws.n, ws.nchunks, static_cast<const typename GT::S*>(demb),
                     bags.batch, tab.num_tables, tab.dim, nv4, static_cast<typename WT::S*>(tab.base),
                     lr, ws.head, ws.tail, ws.through, ws.owner);
  return check_launch("segment_reduce");
}

template <class WT, int LG, int NVG, int S, int LF, int NV>
el_status fixup_t(const el_tables& tab, const GradWorkspace& ws, const uint32_t* keys, float lr,
                  int nv4, hipStream_t stream) {
  hipLaunchKernelGGL((k_seg_blocksum<LF, NV>), dim3(blocks_for(ws.nblk, 4)), dim3(256), 0, stream,
                     static_cast<const float*>(ws.head), static_cast<const uint32_t*>(ws.through),
                     ws.nchunks, ws.nblk, tab.dim, nv4, ws.bsum, ws.bthrough);
  el_status st = check_launch("segment_blocksum");
  if (st != EL_OK) return st;
  hipLaunchKernelGGL((k_seg_fixup<WT, LG, NVG, S, LF, NV>), dim3(blocks_for(ws.nchunks, 4 * kFixChunks)), dim3(256),
                     0, stream,
                     keys, ws.n, ws.nchunks, tab.dim, nv4, static_cast<typename WT::S*>(tab.base), lr,
                     static_cast<const float*>(ws.head), static_cast<const float*>(ws.tail),
                     static_cast<const uint32_t*>(ws.through), static_cast<const uint32_t*>(ws.owner),
                     static_cast<const float*>(ws.bsum), static_cast<const uint32_t*>(ws.bthrough),
                     ws.nblk);
  return check_launch("segment_fixup");
}

template <class GT, class WT>
el_status reduce_typed(const el_tables& tab, const el_bags& bags, const GradWorkspace& ws,
                       const uint32_t* keys, const uint32_t* vals, const void* demb, float lr,
                       hipStream_t stream) {
  // rows split into 4-element vectors; chunk groups need at least 16 lanes (one row number
  // per lane), so narrow rows leave lanes idle
  const int nv4 = tab.dim / 4;
  el_status st;
  if (nv4 <= 16) st = chunk_t<GT, WT, 16, 1>(tab, bags, ws, keys, vals, demb, lr, nv4, stream);
  else if (nv4 <= 32) st = chunk_t<GT, WT, 32, 1>(tab, bags, ws, keys, vals, demb, lr, nv4, stream);
  else if (nv4 <= 64) st = chunk_t<GT, WT, 64, 1>(tab, bags, ws, keys, vals, demb, lr, nv4, stream);
  else if (nv4 <= 128) st = chunk_t<GT, WT, 64, 2>(tab, bags, ws, keys, vals, demb, lr, nv4, stream);
  else return set_error(EL_ERR_UNSUPPORTED, "emb_grad_reduce_update: dim > 512 is not supported");
  if (st != EL_OK) return st;
  // fix-up: short runs by groups of LG lanes (NVG vectors each, S head partials in flight),
  // long runs by the wavefront (LF lanes per row, NV vectors each)
  if (nv4 <= 1) return fixup_t<WT, 1, 1, 8, 1, 1>(tab, ws, keys, lr, nv4, stream);
  if (nv4 <= 2) return fixup_t<WT, 2, 1, 8, 2, 1>(tab, ws, keys, lr, nv4, stream);
  if (nv4 <= 4) return fixup_t<WT, 4, 1, 8, 4, 1>(tab, ws, keys, lr, nv4, stream);
  if (nv4 <= 8) return fixup_t<WT, 8, 1, 8, 8, 1>(tab, ws, keys, lr, nv4, stream);
  if (nv4 <= 16) return fixup_t<WT, 16, 1, 8, 16, 1>(tab, ws, keys, lr, nv4, stream);
  if (nv4 <= 32) return fixup_t<WT, 16, 2, 8, 32, 1>(tab, ws, keys, lr, nv4, stream);
  if (nv4 <= 64) return fixup_t<WT, 16, 4, 4, 64, 1>(tab, ws, keys, lr, nv4, stream);
  return fixup_t<WT, 32, 4, 4, 64, 2>(tab, ws, keys, lr, nv4, stream);
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
  if (tab.dim % 4 != 0)
    return set_error(EL_ERR_UNSUPPORTED, "emb_grad_reduce_update: dim must be a multiple of 4");
  switch (grad_dtype) {
    case EL_F32: return reduce_w<F32T>(tab, bags, ws, sorted_keys, sorted_vals, demb, lr, stream);
    case EL_F16: return reduce_w<F16T>(tab, bags, ws, sorted_keys, sorted_vals, demb, lr, stream);
    case EL_BF16: return reduce_w<BF16T>(tab, bags, ws, sorted_keys, sorted_vals, demb, lr, stream);
  }
  return set_error(EL_ERR_INVALID_ARG, "unknown gradient dtype");
}

}  // namespace el
