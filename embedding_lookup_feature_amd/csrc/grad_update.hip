// grad_update.hip -- segment reduce of the sorted embedding gradients and the SGD row
// update (gfx950).
//
// Plain SGD on the embedding rows (page "DLRM For PyTorch", §Command-line options --lr):
// W[r] <- W[r] - lr * (sum of the gradients of all lookups of row r).  The lookups arrive
// sorted by row (grad_sort.hip), so the contributions to one row form a run.
//
// Skewed (Zipf) indices make some runs thousands of lookups long, so the work is cut by
// sorted position, not by run:
//   k_seg_reduce: a workgroup takes a range of G * CH consecutive sorted lookups, each of
//     its G lane groups (L lanes, EPL elements of a row per lane) CH of them (16, or 32 for
//     multi-hot bags), in batches of SUB.  A group issues a batch's gradient-row loads, and
//     the table-row loads of the runs that end in it, before any store; it sums its lookups
//     in order (fp32), one "piece" per run, and updates the rows of the runs that lie inside
//     its CH lookups.  A piece that continues into the next group's lookups goes to an LDS
//     slot.  After one barrier the group where such a run ends adds the earlier groups'
//     slots in group order, then its own piece, and updates the row.  Only runs that cross
//     an edge of the workgroup's range
//     leave an fp32 partial row in HBM: the run coming in from the previous range (its
//     pieces in this range: the range's "head"; the whole range if one run covers it) and
//     the run going out to the next range (the range's "tail").
//   k_seg_fixup: one lane group per range whose last run continues into later ranges: the
//     tail partial plus the head partials of the following ranges up to the one where the
//     run ends, in range order, then the row update.
// Every sum has a fixed association (lookups in sorted order within a piece, pieces in
// group order within a range, partials in range order across ranges), so results are
// bitwise reproducible; nothing uses atomics and every row is written by one lane group.
// Loads and stores share one completion counter on this architecture, so a group issues
// every load it needs before its first store.
#include <type_traits>

#include "el_internal.hpp"

namespace el {
namespace {

constexpr uint32_t NONE = 0xffffffffu;  // not a row: rows are < total_rows < 2^32 - 1
constexpr uint32_t RANGE_THROUGH = 1u;  // one run covers the whole range
constexpr uint32_t RANGE_OWNER = 2u;    // the range's last run continues into the next range

// N consecutive elements of T as raw 32-bit words (8, 16 or 32 bytes), loaded unconverted
// so that issuing the load never waits.
template <class T, int N>
struct Raw {
  static constexpr int NW = N * static_cast<int>(sizeof(typename T::S)) / 4;
  uint32_t w[NW];
};

// Element offset of row r of a row-major matrix of D-element rows (one 32 x 32 -> 64-bit
// multiply: r and D are non-negative).
__device__ inline uint64_t row_off(uint32_t r, int D) {
  return static_cast<uint64_t>(r) * static_cast<uint32_t>(D);
}

template <class T, int N>
__device__ inline Raw<T, N> load_raw(const typename T::S* p) {
  Raw<T, N> r;
  if constexpr (Raw<T, N>::NW == 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    r.w[0] = v.x; r.w[1] = v.y;
  } else {
#pragma unroll
    for (int i = 0; i < Raw<T, N>::NW / 4; ++i) {
      const uint4 v = reinterpret_cast<const uint4*>(p)[i];
      r.w[4 * i] = v.x; r.w[4 * i + 1] = v.y; r.w[4 * i + 2] = v.z; r.w[4 * i + 3] = v.w;
    }
  }
  return r;
}

// The same, non-temporal: every table row the update touches is read once and written
// once; a gradient row too when bags hold one lookup (a multi-hot bag's gradient row is
// read once per lookup of the bag, and is then left to the cache).
typedef uint32_t nt_u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t nt_u32x4 __attribute__((ext_vector_type(4)));

template <class T, int N>
__device__ inline Raw<T, N> load_raw_nt(const typename T::S* p) {
  Raw<T, N> r;
  if constexpr (Raw<T, N>::NW == 2) {
    const nt_u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x2*>(p));
    r.w[0] = v.x; r.w[1] = v.y;
  } else {
#pragma unroll
    for (int i = 0; i < Raw<T, N>::NW / 4; ++i) {
      const nt_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4*>(p) + i);
      r.w[4 * i] = v.x; r.w[4 * i + 1] = v.y; r.w[4 * i + 2] = v.z; r.w[4 * i + 3] = v.w;
    }
  }
  return r;
}

template <class T, int N>
__device__ inline void raw_to_f(const Raw<T, N>& r, float* f) {
  if constexpr (sizeof(typename T::S) == 4) {
#pragma unroll
    for (int i = 0; i < N; ++i) f[i] = __uint_as_float(r.w[i]);
  } else {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      f[2 * i] = T::to_f(static_cast<uint16_t>(r.w[i] & 0xffffu));
      f[2 * i + 1] = T::to_f(static_cast<uint16_t>(r.w[i] >> 16));
    }
  }
}

// W[i] <- round(W[i] - lr * g[i]) for N elements at w, from the loaded old values (fp32
// FMA, one rounding).
template <class WT, int N>
__device__ inline void sgd_store(typename WT::S* w, const Raw<WT, N>& old, const float* g, float lr) {
  float cur[N];
  raw_to_f<WT, N>(old, cur);
#pragma unroll
  for (int i = 0; i < N; ++i) cur[i] = fmaf(-lr, g[i], cur[i]);
  // non-temporal stores of the rounded row (see load_raw_nt)
  constexpr int NW = Raw<WT, N>::NW;
  uint32_t wd[NW];
  if constexpr (sizeof(typename WT::S) == 4) {
#pragma unroll
    for (int i = 0; i < N; ++i) wd[i] = __float_as_uint(cur[i]);
  } else {
#pragma unroll
    for (int i = 0; i < N / 2; ++i)
      wd[i] = static_cast<uint32_t>(WT::from_f(cur[2 * i])) | (static_cast<uint32_t>(WT::from_f(cur[2 * i + 1])) << 16);
  }
  if constexpr (NW == 2) {
    __builtin_nontemporal_store(nt_u32x2{wd[0], wd[1]}, reinterpret_cast<nt_u32x2*>(w));
  } else {
#pragma unroll
    for (int i = 0; i < NW / 4; ++i)
      __builtin_nontemporal_store(nt_u32x4{wd[4 * i], wd[4 * i + 1], wd[4 * i + 2], wd[4 * i + 3]},
                                  reinterpret_cast<nt_u32x4*>(w) + i);
  }
}

// First local position i in [0, hi] of the range with key(i) == k (k occurs at hi).
__device__ inline int first_of(const uint32_t* skey, uint32_t k, int hi) {
  int lo = 0;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (skey[1 + mid] < k) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// GT: gradient type, WT: table type; L lanes per row (a power of two), EPL elements per lane,
// CH lookups per lane group, SUB of them loaded at once; GNT: gradient rows non-temporal.
template <class GT, class WT, int L, int EPL, int CH, int SUB, bool GNT>
__global__ __launch_bounds__(256) void k_seg_reduce(
    const uint32_t* __restrict__ keys, const uint32_t* __restrict__ vals, int64_t n,
    const typename GT::S* __restrict__ demb, int32_t B, int32_t F, int32_t D,
    typename WT::S* __restrict__ W, float lr, float* __restrict__ rhead,
    float* __restrict__ rtail, uint32_t* __restrict__ rflags, int64_t nranges) {
  constexpr int G = 256 / L;       // lane groups per workgroup
  constexpr int RANGE = G * CH;    // sorted lookups per workgroup
  constexpr int PITCH = L * EPL;   // floats per LDS slot (>= D)
  __shared__ uint32_t skey[RANGE + 2];  // key before the range, the range's keys, key after
  __shared__ uint32_t sval[RANGE];      // gradient row (b * F + t) of each lookup's bag
  __shared__ float slot[G * PITCH];     // per group: the piece that continues past its lookups

  const int tid = threadIdx.x;
  const int g = tid / L, gl = tid % L;
  // each XCD takes one contiguous run of ranges, so that the gradient rows its lookups
  // re-read (the bags of the few tables it is working on) stay in its L2
  const int64_t w = xcd_remap(blockIdx.x, gridDim.x);
  if (w >= nranges) return;  // the grid is rounded up to a multiple of 8 (whole workgroup)
  const int64_t p0 = w * RANGE;
  const int nloc = static_cast<int>(n - p0 < RANGE ? n - p0 : RANGE);  // lookups of the range, >= 1

  // keys and bag ids of the range, and the keys on either side of it (NONE past the ends)
  for (int i = tid; i < RANGE; i += 256) {
    const bool ok = i < nloc;
    skey[1 + i] = ok ? ld_stream(keys + p0 + i) : NONE;
    // bag t * B + b -> its row of demb, b * F + t (< F * B < 2^31), once per lookup here
    // rather than in each lane that loads the row
    const uint32_t bag = ok ? ld_stream(vals + p0 + i) : 0u;
    const uint32_t t = bag / static_cast<uint32_t>(B);
    sval[i] = (bag - t * static_cast<uint32_t>(B)) * static_cast<uint32_t>(F) + t;
  }
  if (tid == 0) skey[0] = p0 > 0 ? keys[p0 - 1] : NONE;
  if (tid == 1) skey[RANGE + 1] = p0 + RANGE < n ? keys[p0 + RANGE] : NONE;
  __syncthreads();

  const int c0 = g * CH;  // first lookup of this group (local)
  const int cnt = nloc - c0 <= 0 ? 0 : (nloc - c0 < CH ? nloc - c0 : CH);
  const int e0 = gl * EPL < D ? gl * EPL : 0;  // this lane's first element (idle lanes: 0)
  const bool lane_on = gl * EPL < D;
  const uint32_t kbefore = skey[0];  // key before the range

  float hacc[EPL];        // the group's head piece (a run that began in an earlier group)
  Raw<WT, EPL> whead;     // and its table row, when the run began inside the range
  bool has_head = false;  // group-uniform
#pragma unroll
  for (int x = 0; x < EPL; ++x) hacc[x] = 0.0f;
#pragma unroll
  for (int x = 0; x < Raw<WT, EPL>::NW; ++x) whead.w[x] = 0u;

  if (cnt > 0) {  // group-uniform
    const uint32_t khead = skey[1 + c0];
    const bool head_cont = khead == skey[c0];  // the first run began before this group
    float acc[EPL];
#pragma unroll
    for (int x = 0; x < EPL; ++x) acc[x] = 0.0f;
    // the group's lookups in batches of SUB (fewer rows held in registers at once); the
    // running piece carries over from one batch to the next
#pragma unroll 1
    for (int qb = 0; qb < cnt; qb += SUB) {
      const int hc = cnt - qb < SUB ? cnt - qb : SUB;  // lookups of this batch
      uint32_t kq[SUB + 1];
#pragma unroll
      for (int q = 0; q <= SUB; ++q) kq[q] = skey[1 + c0 + qb + (q < hc ? q : hc)];  // kq[hc..]: key after

      // (1) every load of the batch: its gradient rows (positions past the end re-read the
      //     last one), and the table rows of the runs that end here and began inside the
      //     range (a run that began before the range is finished by the fix-up)
      Raw<GT, EPL> gr[SUB];
      Raw<WT, EPL> wold[SUB];
#pragma unroll
      for (int q = 0; q < SUB; ++q) {
        const uint32_t grow = sval[c0 + qb + (q < hc ? q : hc - 1)];
        const typename GT::S* gsrc = demb + row_off(grow, D) + e0;
        if constexpr (GNT) gr[q] = load_raw_nt<GT, EPL>(gsrc);
        else gr[q] = load_raw<GT, EPL>(gsrc);
      }
#pragma unroll
      for (int q = 0; q < SUB; ++q) {
#pragma unroll
        for (int x = 0; x < Raw<WT, EPL>::NW; ++x) wold[q].w[x] = 0u;
        // a run ends at lookup q (never at q >= hc: kq[hc..SUB] all hold the key after)
        if (kq[q] != kq[q + 1] && kq[q] != kbefore) wold[q] = load_raw_nt<WT, EPL>(W + row_off(kq[q], D) + e0);
      }

      // (2) pieces in order: a run inside the group is finished here; the head piece waits
      //     for the barrier; the last piece, if it continues, goes to the group's slot
#pragma unroll
      for (int q = 0; q < SUB; ++q) {
        if (q < hc) {
          float f[EPL];
          raw_to_f<GT, EPL>(gr[q], f);
#pragma unroll
          for (int x = 0; x < EPL; ++x) acc[x] += f[x];
          const bool ends = kq[q] != kq[q + 1];           // a piece ends here
          const bool head = ends && head_cont && kq[q] == khead;
          if (ends && !head && lane_on) sgd_store<WT, EPL>(W + row_off(kq[q], D) + e0, wold[q], acc, lr);
#pragma unroll
          for (int x = 0; x < EPL; ++x) hacc[x] = head ? acc[x] : hacc[x];
#pragma unroll
          for (int x = 0; x < Raw<WT, EPL>::NW; ++x) whead.w[x] = head ? wold[q].w[x] : whead.w[x];
          has_head = has_head || head;
#pragma unroll
          for (int x = 0; x < EPL; ++x) acc[x] = ends ? 0.0f : acc[x];
        }
      }
    }
    if (skey[c0 + cnt] == skey[1 + c0 + cnt]) {  // the last piece continues past this group
#pragma unroll
      for (int x = 0; x < EPL; ++x) slot[g * PITCH + gl * EPL + x] = acc[x];
    }
  }
  __syncthreads();

  // (3) runs that cross group edges: the group where such a run ends adds the slots of the
  //     groups before it (in group order) and its own piece
  if (has_head) {
    const uint32_t kh = skey[1 + c0];
    const int cf = first_of(skey, kh, c0) / CH;  // group where the run's first piece lies
    float tot[EPL];
#pragma unroll
    for (int x = 0; x < EPL; ++x) tot[x] = 0.0f;
    for (int c = cf; c < g; ++c) {
#pragma unroll
      for (int x = 0; x < EPL; ++x) tot[x] += slot[c * PITCH + gl * EPL + x];
    }
#pragma unroll
    for (int x = 0; x < EPL; ++x) tot[x] += hacc[x];
    if (lane_on) {
      if (kh == kbefore)  // began before the range: its part in this range is the head partial
        store_n<F32T, EPL>(rhead + w * D + e0, tot);
      else
        sgd_store<WT, EPL>(W + row_off(kh, D) + e0, whead, tot, lr);
    }
  }
  //     the run that continues past the range: its pieces here are the range's tail partial
  //     (or, if one run covers the whole range, its head partial)
  const int glast = (nloc - 1) / CH;
  const uint32_t klast = skey[nloc];
  const bool cont = klast == skey[1 + nloc];  // NONE past the end of the lookups
  if (g == glast && cont) {
    const int cf = first_of(skey, klast, nloc - 1) / CH;
    float tot[EPL];
#pragma unroll
    for (int x = 0; x < EPL; ++x) tot[x] = 0.0f;
    for (int c = cf; c <= g; ++c) {
#pragma unroll
      for (int x = 0; x < EPL; ++x) tot[x] += slot[c * PITCH + gl * EPL + x];
    }
    if (lane_on) store_n<F32T, EPL>((klast == kbefore ? rhead : rtail) + w * D + e0, tot);
  }
  if (tid == 0) {
    const bool through = cont && klast == kbefore;
    rflags[w] = (through ? RANGE_THROUGH : 0u) | (cont && !through ? RANGE_OWNER : 0u);
  }
}

// One lane group (LF lanes, NV 16-byte vectors of fp32 partials per lane) per range: if the
// range's last run continues into later ranges, add its tail partial and the head partials
// of the following ranges (those one run covers, then the one where it ends) in range
// order, and update the row.  K partials in flight (the hottest rows' runs cross tens of
// ranges, and their chains are the kernel's critical path).
template <class WT, int LF, int NV>
__global__ __launch_bounds__(256) void k_seg_fixup(
    const uint32_t* __restrict__ keys, int64_t n, int64_t nranges, int32_t range, int32_t D,
    typename WT::S* __restrict__ W, float lr, const float* __restrict__ rhead,
    const float* __restrict__ rtail, const uint32_t* __restrict__ rflags) {
  constexpr int K = 8;
  constexpr int FL = 64 / LF;  // flags per lane per scan step: 64 per group
  const int gl = threadIdx.x % LF;
  const int64_t w = static_cast<int64_t>(blockIdx.x) * (256 / LF) + threadIdx.x / LF;
  if (w >= nranges || !(rflags[w] & RANGE_OWNER)) return;  // group-uniform
  const int64_t last = (w + 1) * range < n ? (w + 1) * range : n;
  const uint32_t key = keys[last - 1];
  // the range where the run ends: the first one after w that one run does not cover (the
  // last range is never covered); 64 flags per step, the group's first hit by ballot
  const int lane = threadIdx.x & 63;
  const int gbase = lane - gl;
  int64_t e = w + 1;
  for (;;) {
    int hit = FL;
#pragma unroll
    for (int j = FL - 1; j >= 0; --j) {
      const int64_t i = e + static_cast<int64_t>(gl) * FL + j;
      if (i >= nranges || !(rflags[i] & RANGE_THROUGH)) hit = j;
    }
    const uint64_t m = (__ballot(hit < FL) >> gbase) & (LF == 64 ? ~0ull : ((1ull << LF) - 1ull));
    if (m) {
      const int first = __ffsll(static_cast<unsigned long long>(m)) - 1;  // group lane
      e += static_cast<int64_t>(first) * FL + __shfl(hit, gbase + first);
      break;
    }
    e += 64;
  }
  float tot[NV][4];
  Raw<WT, 4> wold[NV];
#pragma unroll
  for (int m = 0; m < NV; ++m) {
    const int v = gl + m * LF;
    const int vo = (v * 4 < D ? v : 0) * 4;
    wold[m] = load_raw_nt<WT, 4>(W + static_cast<int64_t>(key) * D + vo);
    const uint4 t = *reinterpret_cast<const uint4*>(rtail + w * D + vo);
    tot[m][0] = __uint_as_float(t.x); tot[m][1] = __uint_as_float(t.y);
    tot[m][2] = __uint_as_float(t.z); tot[m][3] = __uint_as_float(t.w);
  }
  for (int64_t r0 = w + 1; r0 <= e; r0 += K) {
    uint4 h[K][NV];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int64_t r = r0 + k <= e ? r0 + k : e;
#pragma unroll
      for (int m = 0; m < NV; ++m) {
        const int v = gl + m * LF;
        h[k][m] = *reinterpret_cast<const uint4*>(rhead + r * D + (v * 4 < D ? v : 0) * 4);
      }
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
      if (r0 + k <= e) {
#pragma unroll
        for (int m = 0; m < NV; ++m) {
          tot[m][0] += __uint_as_float(h[k][m].x); tot[m][1] += __uint_as_float(h[k][m].y);
          tot[m][2] += __uint_as_float(h[k][m].z); tot[m][3] += __uint_as_float(h[k][m].w);
        }
      }
    }
  }
#pragma unroll
  for (int m = 0; m < NV; ++m) {
    const int v = gl + m * LF;
    if (v * 4 < D) sgd_store<WT, 4>(W + static_cast<int64_t>(key) * D + v * 4, wold[m], tot[m], lr);
  }
}

int blocks_for(int64_t n, int per) { return static_cast<int>((n + per - 1) / per); }

template <class GT, class WT, int L, int EPL>
el_status reduce_t(const el_tables& tab, const el_bags& bags, const GradWorkspace& ws,
                   const uint32_t* keys, const uint32_t* vals, const void* demb, float lr,
                   hipStream_t stream) {
  // at most one lookup per bag on average: every gradient row is read about once, so it is
  // streamed (non-temporal) like the table rows; otherwise a bag's row is re-read once per
  // lookup and is left to the cache
  const bool once = ws.n <= static_cast<int64_t>(bags.batch) * tab.num_tables;
  // Lookups per lane group and per load batch, measured on the training-step and multi-hot
  // shapes with both table types.  Rows read once are bandwidth-bound and want bytes in
  // flight: 16 per group, 8 at once (update 147-185 us, against 151-190 with 2 or 4 at once,
  // 157-183 with 16, and 153-190 with 32 per group).  A multi-hot bag's rows come back from
  // L2 and the table rows' latency is what remains, so more resident wavefronts with fewer
  // loads each win, and longer ranges leave fewer partials: 32 per group, 1 at once for
  // 16-bit tables (730 us against 757 with 2 and 923 with 8 of 16) and 4 for fp32 (1076
  // against 1160 with 2 and 1227 with 8 of 16).
  int64_t nr = 0, range = 0;
  auto reduce = [&](auto gnt) {
    constexpr bool GNT = decltype(gnt)::value;
    constexpr int CH = GNT ? kChunk : 2 * kChunk;
    constexpr int SUB = GNT ? 8 : (sizeof(typename WT::S) == 2 ? 1 : 4);
    constexpr int RANGE = (256 / L) * CH;
    static_assert(RANGE >= kMinRange, "the workspace holds partials for ranges of >= kMinRange lookups");
    range = RANGE;
    nr = (ws.n + RANGE - 1) / RANGE;
    hipLaunchKernelGGL((k_seg_reduce<GT, WT, L, EPL, CH, SUB, GNT>),
                       dim3(static_cast<unsigned>(round_up8(nr))), dim3(256), 0, stream, keys, vals, ws.n,
                       static_cast<const typename GT::S*>(demb), bags.batch, tab.num_tables, tab.dim,
                       static_cast<typename WT::S*>(tab.base), lr, ws.range_head, ws.range_tail,
                       ws.range_flags, nr);
  };
  if (once)
    reduce(std::true_type{});
  else
    reduce(std::false_type{});
  el_status st = check_launch("segment_reduce");
  if (st != EL_OK || nr < 2) return st;
  // fix-up: LF lanes x NV vectors of 4 fp32 per row
  const int d4 = tab.dim / 4;
  auto fix = [&](auto lf, auto nv) {
    constexpr int LF = decltype(lf)::value, NV = decltype(nv)::value;
    hipLaunchKernelGGL((k_seg_fixup<WT, LF, NV>), dim3(blocks_for(nr, 256 / LF)), dim3(256), 0, stream,
                       keys, ws.n, nr, static_cast<int>(range), tab.dim, static_cast<typename WT::S*>(tab.base), lr,
                       static_cast<const float*>(ws.range_head), static_cast<const float*>(ws.range_tail),
                       static_cast<const uint32_t*>(ws.range_flags));
    return check_launch("segment_fixup");
  };
  using I = std::integral_constant<int, 1>;
  if (d4 <= 1) return fix(I{}, I{});
  if (d4 <= 2) return fix(std::integral_constant<int, 2>{}, I{});
  if (d4 <= 4) return fix(std::integral_constant<int, 4>{}, I{});
  if (d4 <= 8) return fix(std::integral_constant<int, 8>{}, I{});
  if (d4 <= 16) return fix(std::integral_constant<int, 16>{}, I{});
  if (d4 <= 32) return fix(std::integral_constant<int, 32>{}, I{});
  if (d4 <= 64) return fix(std::integral_constant<int, 64>{}, I{});
  return fix(std::integral_constant<int, 64>{}, std::integral_constant<int, 2>{});
}

// Elements per lane: 4 (8- or 16-byte parts of the rows: sixteen of each in flight per lane
// keep the registers low enough for three or more wavefronts per SIMD); lanes per row: the
// power of two that covers D.
template <class GT, class WT>
el_status reduce_typed(const el_tables& tab, const el_bags& bags, const GradWorkspace& ws,
                       const uint32_t* keys, const uint32_t* vals, const void* demb, float lr,
                       hipStream_t stream) {
  constexpr int EPL = 4;
  if (tab.dim % EPL != 0)
    return set_error(EL_ERR_UNSUPPORTED, "emb_grad_reduce_update: dim must be a multiple of 16 bytes of both row types");
  // 16-bit gradient and table rows: 8 elements (16 bytes of each) per lane, so that a
  // workgroup's lane groups cover twice the lookups with the same number of loads
  if constexpr (sizeof(typename GT::S) == 2 && sizeof(typename WT::S) == 2) {
    const int l8 = tab.dim / 8;
    if (tab.dim % 8 == 0 && l8 >= 4 && l8 <= 64) {
      if (l8 <= 4) return reduce_t<GT, WT, 4, 8>(tab, bags, ws, keys, vals, demb, lr, stream);
      if (l8 <= 8) return reduce_t<GT, WT, 8, 8>(tab, bags, ws, keys, vals, demb, lr, stream);
      if (l8 <= 16) return reduce_t<GT, WT, 16, 8>(tab, bags, ws, keys, vals, demb, lr, stream);
      if (l8 <= 32) return reduce_t<GT, WT, 32, 8>(tab, bags, ws, keys, vals, demb, lr, stream);
      return reduce_t<GT, WT, 64, 8>(tab, bags, ws, keys, vals, demb, lr, stream);
    }
  }
  const int lanes = tab.dim / EPL;
  if constexpr (EPL == 4) {  // rows of more than 64 vectors: 8 elements per lane
    if (lanes > 64 && tab.dim % 8 == 0 && tab.dim <= 512)
      return reduce_t<GT, WT, 64, 8>(tab, bags, ws, keys, vals, demb, lr, stream);
  }
  if (lanes <= 1) return reduce_t<GT, WT, 1, EPL>(tab, bags, ws, keys, vals, demb, lr, stream);
  if (lanes <= 2) return reduce_t<GT, WT, 2, EPL>(tab, bags, ws, keys, vals, demb, lr, stream);
  if (lanes <= 4) return reduce_t<GT, WT, 4, EPL>(tab, bags, ws, keys, vals, demb, lr, stream);
  if (lanes <= 8) return reduce_t<GT, WT, 8, EPL>(tab, bags, ws, keys, vals, demb, lr, stream);
  if (lanes <= 16) return reduce_t<GT, WT, 16, EPL>(tab, bags, ws, keys, vals, demb, lr, stream);
  if (lanes <= 32) return reduce_t<GT, WT, 32, EPL>(tab, bags, ws, keys, vals, demb, lr, stream);
  if (lanes <= 64) return reduce_t<GT, WT, 64, EPL>(tab, bags, ws, keys, vals, demb, lr, stream);
  return set_error(EL_ERR_UNSUPPORTED, "emb_grad_reduce_update: dim > 512 is not supported");
}

template <class GT>
el_status reduce_w(const el_tables& tab, const el_bags& bags, const GradWorkspace& ws,
                   const uint32_t* keys, const uint32_t* vals, const void* demb, float lr,
                   hipStream_t stream) {
  switch (tab.dtype) {
    case EL_F32: return reduce_typed<GT, F32T>(tab, bags, ws, keys, vals, demb, lr, stream);
    case EL_F16: return reduce_typed<GT, F16T>(tab, bags, ws, keys, vals, demb, lr, stream);
    case EL_BF16: return reduce_typed<GT, BF16T>(tab, bags, ws, keys, vals, demb, lr, stream);
    default: break;
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
    default: break;
  }
  return set_error(EL_ERR_INVALID_ARG, "unknown gradient dtype");
}

}  // namespace el
