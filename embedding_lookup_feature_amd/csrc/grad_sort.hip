// grad_sort.hip -- the embedding-gradient lookups sorted by row: stable LSD radix sort of
// each table's lookups by local row, run-length segments, and the exclusive scan they use
// (gfx950).
//
// Every lookup k of bag g = t*B + b contributes demb[b][t] to row row_offset[t] + idx[k]
// of the joint table (plain SGD, page "DLRM For PyTorch", §Command-line options --lr).
// Sorting the (row, bag) pairs by row puts all contributions to one row next to each
// other, so that the reduction needs no atomics.
//
// The lookups are table-major (table t's lookups are the positions of bags t*B .. t*B+B-1)
// and table t's rows are the joint rows [row_offset[t], row_offset[t+1]), so sorting every
// table's run of lookups by local row, in place, sorts the whole array by joint row: the
// sort works on local rows, whose width is that of the largest table (max_rows) instead of
// that of all rows together, and adds the table's first row when it writes the last pass.
//
// Radix sort: least significant digit first, the fewest passes of at most kRadixBits-bit
// digits that cover the local rows, with equal digit widths (20-bit rows: 3 x 7 bits;
// 17-bit rows: 2 x 9 bits).
// Tiles of 4096 keys never straddle two tables (a table's last tile may be short).  One
// pass = tile histograms -> per digit, a scan over the tiles -> stable scatter; the scatter
// takes its table's digit starts from the scanned counts at the table's first and last
// tiles.  The first pass reads the indices themselves (and the bag ids written once by
// k_build_vals), so the local rows are never stored unsorted.  Within a tile, 4 wavefronts
// x 16 steps x 64 lanes, each wavefront owning 1024 consecutive keys; within a step the
// lanes holding the same digit are found with one ballot per digit bit in the scatter; the
// lowest of them adds the group's size to its wavefront's private LDS counter, so every
// counter has one writer per step and the ranks need no atomic.  Ranks are taken in key
// order (wave, step, lane), which makes every pass stable and the whole sort deterministic.
// The tile histograms use integer LDS atomics (exact counts whatever the order of the
// adds).  The ranked tile is staged in LDS in sorted order and written out run by run, so
// that neighbouring threads store to neighbouring addresses.
#include "el_internal.hpp"

namespace el {
namespace {

__device__ inline uint64_t lanemask_lt(int lane) { return (1ull << lane) - 1ull; }

// Lanes of this wavefront whose (valid) RB-bit digit equals this lane's digit.
template <int RB>
__device__ inline uint64_t match_digit(uint32_t d, bool valid) {
  uint64_t m = __ballot(valid);
#pragma unroll
  for (int bit = 0; bit < RB; ++bit) {
    const bool x = (d >> bit) & 1u;
    const uint64_t bb = __ballot(x);
    m &= x ? bb : ~bb;
  }
  return m;
}

// Bag id of every lookup position.  A block takes 256 consecutive bags: their CSR bounds go
// to LDS.  Bags of one lookup each (position k of the block holds bag k - first): every
// position's bag is checked with one probe and written straight away.  Otherwise the
// block's positions are covered in windows of kBagWin: each thread marks the positions of
// its own bag that fall in the window with the bag's number in LDS, and after a barrier the
// block writes the window out with unit stride, so stores are coalesced for any bag lengths.
constexpr int kBagWin = 4096;

__global__ __launch_bounds__(256) void k_build_vals(const int32_t* __restrict__ off, int32_t nbags,
                                                    uint32_t* __restrict__ vals) {
  __shared__ int32_t bound[257];
  __shared__ uint8_t mark[kBagWin];  // bag of the window's positions, relative to the block
  __shared__ int32_t one_each;
  const int g0 = blockIdx.x * 256;
  const int nb = nbags - g0 < 256 ? nbags - g0 : 256;  // bags of this block
  for (int i = threadIdx.x; i <= nb; i += 256) bound[i] = ld_stream(off + g0 + i);
  if (threadIdx.x == 0) one_each = 1;
  __syncthreads();
  const int s = bound[0], e = bound[nb];
  const int t = threadIdx.x;
  if (t < nb && bound[t + 1] - bound[t] != 1) one_each = 0;  // any thread may clear it
  __syncthreads();
  if (one_each) {  // block-uniform
    for (int k = s + t; k < e; k += 256) vals[k] = static_cast<uint32_t>(g0 + (k - s));
    return;
  }
  const int bs = t < nb ? bound[t] : 0, be = t < nb ? bound[t + 1] : 0;  // this thread's bag
  for (int w0 = s; w0 < e; w0 += kBagWin) {  // block-uniform
    const int w1 = e - w0 < kBagWin ? e : w0 + kBagWin;
    for (int k = bs > w0 ? bs : w0; k < (be < w1 ? be : w1); ++k) mark[k - w0] = static_cast<uint8_t>(t);
    __syncthreads();
    for (int k = w0 + t; k < w1; k += 256) vals[k] = static_cast<uint32_t>(g0 + mark[k - w0]);
    __syncthreads();  // the window's marks are read before the next window's are written
  }
}

// Exclusive scan of x over the 256 threads of a block (every thread gets its prefix; `total`
// receives the block sum).  `wsum` is 4 words of LDS.
__device__ inline uint32_t block_exclusive_scan(uint32_t x, uint32_t* wsum, uint32_t& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t inc = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(inc, o);
    if (lane >= o) inc += y;
  }
  if (lane == 63) wsum[w] = inc;
  __syncthreads();
  uint32_t pre = 0;
  for (int i = 0; i < w; ++i) pre += wsum[i];
  total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  __syncthreads();  // wsum is reused by the next call
  return pre + inc - x;
}

// Tiles of the sort: table t's lookups (positions offsets[t*B] .. offsets[t*B+B]) are cut
// into ceil(len / kSortTile) tiles, so that no tile holds two tables' lookups;
// tile_prefix[t] = tiles of the tables before t (tile_prefix[F] = all tiles).  One block,
// 256 tables per step.
__global__ __launch_bounds__(256) void k_sort_tiles(const int32_t* __restrict__ off, int32_t B,
                                                    int32_t F, int32_t* __restrict__ tile_prefix) {
  __shared__ uint32_t wsum[4];
  uint32_t carry = 0;
  for (int t0 = 0; t0 <= F; t0 += 256) {
    const int t = t0 + static_cast<int>(threadIdx.x);
    uint32_t nt = 0;
    if (t < F) {
      const int32_t s = off[static_cast<int64_t>(t) * B], e = off[static_cast<int64_t>(t + 1) * B];
      nt = e > s ? static_cast<uint32_t>((e - s + kSortTile - 1) / kSortTile) : 0u;
    }
    uint32_t total;
    const uint32_t pre = block_exclusive_scan(nt, wsum, total);
    if (t <= F) tile_prefix[t] = static_cast<int32_t>(carry + pre);
    carry += total;
  }
}

// Where every tile's keys are: tile j belongs to the last table t with tile_prefix[t] <= j
// (tables without lookups own no tile); tiles past the last one (the grid is sized for the
// most tiles any split can give) hold no keys.
__global__ __launch_bounds__(256) void k_tile_info(const int32_t* __restrict__ off, int32_t B, int32_t F,
                                                   const int32_t* __restrict__ tile_prefix, int32_t nblocks,
                                                   SortTile* __restrict__ tiles) {
  const int j = static_cast<int>(blockIdx.x) * 256 + static_cast<int>(threadIdx.x);
  if (j >= nblocks) return;
  int lo = 0, hi = F;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tile_prefix[mid] <= j) lo = mid; else hi = mid - 1;
  }
  SortTile ti{0, 0, 0, 0, 0, 0, 0, 0};
  if (lo < F) {
    const int32_t s = off[static_cast<int64_t>(lo) * B], e = off[static_cast<int64_t>(lo + 1) * B];
    const int32_t start = static_cast<int32_t>(s + static_cast<int64_t>(j - tile_prefix[lo]) * kSortTile);
    ti.t = lo;
    ti.start = start;
    ti.count = e - start < kSortTile ? e - start : kSortTile;
    ti.seg_start = s;
    ti.first = tile_prefix[lo];
    ti.end = tile_prefix[lo + 1];
  }
  tiles[j] = ti;
}

// Local row of lookup p of table t (FIRST pass: straight from the indices).  STREAM: a
// non-temporal load (the scatter's, the sort's last read of the indices).
template <bool STREAM = false>
__device__ inline uint32_t local_row(const int32_t* __restrict__ idx, int64_t p, bool hash, int32_t rows) {
  int32_t r = STREAM ? ld_stream(idx + p) : idx[p];
  if (hash) r = floor_mod(r, rows);
  return static_cast<uint32_t>(r);
}

// Digit counts of one tile.  Integer LDS atomics into kSub sub-histograms (wavefront and
// lane group), so that few lanes contend for one counter even when a tile holds many equal
// keys (the hot rows of skewed indices); counts do not depend on the order of the adds, so
// the histograms, and the sort, are deterministic.  (Measured and not kept: counting with
// ballots as the scatter ranks, 1.7-2x slower; several tiles per workgroup; one add per run
// of equal digits in neighbouring lanes.)  FIRST: the keys are the local rows of the
// indices.
template <int RB, bool FIRST>
__global__ __launch_bounds__(256) void k_radix_hist(const uint32_t* __restrict__ keys,
                                                    const int32_t* __restrict__ idx,
                                                    const SortTile* __restrict__ tiles,
                                                    const int64_t* __restrict__ row_off, int hash,
                                                    int shift, uint32_t* __restrict__ hist, int nblocks) {
  constexpr int kRadix = 1 << RB;
  constexpr int kSteps = kSortTile / 256;
  constexpr int kLaneGroups = RB <= 8 ? 8 : 2;  // sub-histograms per wavefront (LDS-bound)
  constexpr int kSub = 4 * kLaneGroups;
  // one pad word per sub-histogram: a digit's counters in the different sub-histograms
  // then fall in different LDS banks
  __shared__ uint32_t cnt[kSub][kRadix + 1];
  for (int i = threadIdx.x; i < kSub * (kRadix + 1); i += 256) (&cnt[0][0])[i] = 0;
  __syncthreads();
  const SortTile ti = tiles[blockIdx.x];
  const int sub = (threadIdx.x >> 6) * kLaneGroups + (threadIdx.x & 63) % kLaneGroups;
  int32_t rows = 0;
  if (FIRST && hash) rows = static_cast<int32_t>(row_off[ti.t + 1] - row_off[ti.t]);
  uint32_t kk[kSteps];
#pragma unroll
  for (int st = 0; st < kSteps; ++st) {
    const int p = static_cast<int>(threadIdx.x) + st * 256;
    if (FIRST)
      kk[st] = p < ti.count ? local_row(idx, static_cast<int64_t>(ti.start) + p, hash, rows) : 0u;
    else
      kk[st] = p < ti.count ? keys[static_cast<int64_t>(ti.start) + p] : 0u;
  }
#pragma unroll
  for (int st = 0; st < kSteps; ++st)
    if (static_cast<int>(threadIdx.x) + st * 256 < ti.count)
      atomicAdd(&cnt[sub][(kk[st] >> shift) & (kRadix - 1)], 1u);
  __syncthreads();
  for (int dg = threadIdx.x; dg < kRadix; dg += 256) {
    uint32_t c = 0;
#pragma unroll
    for (int k = 0; k < kSub; ++k) c += cnt[k][dg];
    hist[static_cast<int64_t>(dg) * nblocks + blockIdx.x] = c;
  }
}

// One block per digit: exclusive scan of that digit's tile counts (tile order), and the
// digit's total.
__global__ __launch_bounds__(256) void k_digit_scan(const uint32_t* __restrict__ hist,
                                                    uint32_t* __restrict__ hist_scan, int nblocks,
                                                    uint32_t* __restrict__ totals) {
  __shared__ uint32_t wsum[4];
  const int64_t row = static_cast<int64_t>(blockIdx.x) * nblocks;
  uint32_t carry = 0;
  for (int b0 = 0; b0 < nblocks; b0 += 256 * 8) {
    uint32_t v[8], sum = 0;
    const int first = b0 + threadIdx.x * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[i] = first + i < nblocks ? hist[row + first + i] : 0u;
      sum += v[i];
    }
    uint32_t total;
    uint32_t run = carry + block_exclusive_scan(sum, wsum, total);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (first + i < nblocks) hist_scan[row + first + i] = run;
      run += v[i];
    }
    carry += total;
  }
  if (threadIdx.x == 0) totals[blockIdx.x] = carry;
}

// Stable scatter of one tile, inside its table's run of positions.  The tile's keys are
// first ranked (per-wave LDS counters, one writer per digit group and step), then staged in
// LDS in tile-local sorted order, and finally written out by consecutive threads to
// consecutive positions of each digit's run, so that the global stores are coalesced
// instead of one address per lane.  Thread i owns the DPT consecutive digits
// [i*DPT, (i+1)*DPT) in the digit scans.  With S(d, j) the scanned count of digit d before
// tile j, the table's keys with digit d number S(d, end) - S(d, first), and this tile's
// keys with digit d start at  seg_start + (the table's keys with a smaller digit)
// + S(d, j) - S(d, first).  FIRST: keys are the local rows of the indices.  LAST: the
// keys are written as joint rows (local row + row_off[t]).
template <int RB, bool FIRST>
__global__ __launch_bounds__(256) void k_radix_scatter(const uint32_t* __restrict__ keys_in,
                                                       const int32_t* __restrict__ idx,
                                                       const uint32_t* __restrict__ vals_in,
                                                       const SortTile* __restrict__ tiles,
                                                       const int64_t* __restrict__ row_off, int hash,
                                                       int last, int shift,
                                                       const uint32_t* __restrict__ hist_scan,
                                                       const uint32_t* __restrict__ totals,
                                                       uint32_t* __restrict__ keys_out,
                                                       uint32_t* __restrict__ vals_out, int nblocks) {
  constexpr int kRadix = 1 << RB;
  constexpr int DPT = kRadix > 256 ? kRadix / 256 : 1;  // digits per thread in the scans
  constexpr int kSteps = kSortTile / 256;                // keys per thread
  static_assert(kSortTile <= 65535, "tile-local positions are 16-bit");
  __shared__ uint16_t cnt[4][kRadix];  // per-wave digit counts, then per-wave bases
  __shared__ uint32_t gofs[kRadix];    // global position of tile-local position 0, per digit
  __shared__ uint32_t wsum[4];
  __shared__ uint32_t sk[kSortTile], sv[kSortTile];
  // each XCD takes one contiguous run of tiles: neighbouring tiles write neighbouring parts
  // of every digit's run, whose partly written lines then meet in the same L2
  const int j = xcd_remap(blockIdx.x, gridDim.x);  // the grid is a multiple of 8
  if (j >= nblocks) return;
  const SortTile ti = tiles[j];
  if (ti.count == 0) return;  // a tile past the last one (the whole block leaves)
  for (int i = threadIdx.x; i < 4 * kRadix; i += 256) (&cnt[0][0])[i] = 0;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t tile0 = ti.start;
  const int tn = ti.count;               // keys in the tile
  const int base = w * (kSortTile / 4);  // this wave's keys: [base, base + kSortTile/4)
  int32_t rows = 0;
  if (FIRST && hash) rows = static_cast<int32_t>(row_off[ti.t + 1] - row_off[ti.t]);
  const uint32_t kadd = last ? static_cast<uint32_t>(row_off[ti.t]) : 0u;
  uint32_t kk[kSteps], vv[kSteps], rk[kSteps];
#pragma unroll
  for (int st = 0; st < kSteps; ++st) {
    const int p = base + st * 64 + lane;
    const bool valid = p < tn;
    if (FIRST)
      kk[st] = valid ? local_row<true>(idx, tile0 + p, hash, rows) : 0u;
    else
      kk[st] = valid ? ld_stream(keys_in + tile0 + p) : 0u;  // the pass's last read of them
    vv[st] = valid ? ld_stream(vals_in + tile0 + p) : 0u;
  }
  // global start of each of this thread's digits (see above)
  const int d0 = threadIdx.x * DPT;
  const bool owns = d0 < kRadix;
  uint32_t tglob[DPT];
  {
    uint32_t tot[DPT], sum = 0;
#pragma unroll
    for (int x = 0; x < DPT; ++x) {
      tot[x] = 0u;
      tglob[x] = 0u;
      if (owns) {
        const int64_t row = static_cast<int64_t>(d0 + x) * nblocks;
        const uint32_t sf = hist_scan[row + ti.first];
        const uint32_t se = ti.end < nblocks ? hist_scan[row + ti.end] : totals[d0 + x];
        tot[x] = se - sf;
        tglob[x] = hist_scan[row + j] - sf;
      }
      sum += tot[x];
    }
    uint32_t total;
    uint32_t run = static_cast<uint32_t>(ti.seg_start) + block_exclusive_scan(sum, wsum, total);
#pragma unroll
    for (int x = 0; x < DPT; ++x) {
      tglob[x] += run;
      run += tot[x];
    }
  }
  // rank within the wave, in key order
#pragma unroll
  for (int st = 0; st < kSteps; ++st) {
    const bool valid = base + st * 64 + lane < tn;
    const uint32_t d = (kk[st] >> shift) & (kRadix - 1);
    const uint64_t m = match_digit<RB>(d, valid);
    const uint32_t before = static_cast<uint32_t>(__popcll(m & lanemask_lt(lane)));
    const uint32_t pre = cnt[w][d];  // every lane reads before the group leader writes
    rk[st] = pre + before;
    if (valid && before == 0) cnt[w][d] = static_cast<uint16_t>(pre + __popcll(m));
  }
  __syncthreads();
  // tile-local start of each digit (scan over digits), per-wave bases, global offsets
  {
    uint32_t dc[DPT], sum = 0;
#pragma unroll
    for (int x = 0; x < DPT; ++x) {
      dc[x] = owns ? static_cast<uint32_t>(cnt[0][d0 + x]) + cnt[1][d0 + x] + cnt[2][d0 + x] + cnt[3][d0 + x]
                   : 0u;
      sum += dc[x];
    }
    uint32_t total;
    uint32_t lstart = block_exclusive_scan(sum, wsum, total);
    if (owns) {
#pragma unroll
      for (int x = 0; x < DPT; ++x) {
        uint32_t run = lstart;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) {
          const uint32_t c = cnt[ww][d0 + x];
          cnt[ww][d0 + x] = static_cast<uint16_t>(run);
          run += c;
        }
        gofs[d0 + x] = tglob[x] - lstart;
        lstart += dc[x];
      }
    }
  }
  __syncthreads();
  // stage in tile-local sorted order
#pragma unroll
  for (int st = 0; st < kSteps; ++st) {
    if (base + st * 64 + lane < tn) {
      const uint32_t d = (kk[st] >> shift) & (kRadix - 1);
      const uint32_t loc = cnt[w][d] + rk[st];
      sk[loc] = kk[st];
      sv[loc] = vv[st];
    }
  }
  __syncthreads();
  // consecutive positions of a digit's run go to consecutive global positions
#pragma unroll
  for (int st = 0; st < kSteps; ++st) {
    const int i = st * 256 + threadIdx.x;
    if (i < tn) {
      const uint32_t key = sk[i];
      const uint32_t dst = gofs[(key >> shift) & (kRadix - 1)] + static_cast<uint32_t>(i);
      keys_out[dst] = key + kadd;
      vals_out[dst] = sv[i];
    }
  }
}

// Exclusive scan of one tile of 4096 values (256 threads x 16 consecutive values).
__global__ __launch_bounds__(256) void k_scan_tile(const uint32_t* __restrict__ in,
                                                   uint32_t* __restrict__ out, int64_t n,
                                                   uint32_t* __restrict__ tile_sums) {
  __shared__ uint32_t wsum[4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kScanTile + tid * 16;
  uint32_t v[16];
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    v[i] = base + i < n ? in[base + i] : 0u;
    sum += v[i];
  }
  // inclusive scan of the thread sums inside the wavefront
  uint32_t inc = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(inc, o);
    if (lane >= o) inc += y;
  }
  if (lane == 63) wsum[w] = inc;
  __syncthreads();
  uint32_t wpre = 0;
  for (int i = 0; i < w; ++i) wpre += wsum[i];
  uint32_t run = wpre + inc - sum;  // exclusive prefix of this thread
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (base + i < n) out[base + i] = run;
    run += v[i];
  }
  if (tid == 255) tile_sums[blockIdx.x] = wsum[0] + wsum[1] + wsum[2] + wsum[3];
}

__global__ __launch_bounds__(256) void k_scan_add(uint32_t* __restrict__ out, int64_t n,
                                                  const uint32_t* __restrict__ tile_pre) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) out[i] += tile_pre[i / kScanTile];
}

__global__ __launch_bounds__(256) void k_seg_flags(const uint32_t* __restrict__ keys, int64_t n,
                                                   uint32_t* __restrict__ flags) {
  const int64_t q = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (q < n) flags[q] = (q == 0 || keys[q] != keys[q - 1]) ? 1u : 0u;
}

__global__ __launch_bounds__(256) void k_seg_emit(const uint32_t* __restrict__ keys,
                                                  const uint32_t* __restrict__ flags,
                                                  const uint32_t* __restrict__ flags_scan, int64_t n,
                                                  uint32_t* __restrict__ unique_rows,
                                                  uint32_t* __restrict__ seg_offsets,
                                                  uint32_t* __restrict__ num_unique) {
  const int64_t q = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (q >= n) return;
  if (flags[q]) {
    const uint32_t u = flags_scan[q];
    unique_rows[u] = keys[q];
    seg_offsets[u] = static_cast<uint32_t>(q);
  }
  if (q == n - 1) {
    const uint32_t U = flags_scan[q] + flags[q];
    num_unique[0] = U;
    seg_offsets[U] = static_cast<uint32_t>(n);
  }
}

__global__ void k_seg_empty(uint32_t* seg_offsets, uint32_t* num_unique) {
  if (threadIdx.x == 0) {
    seg_offsets[0] = 0;
    num_unique[0] = 0;
  }
}

int blocks_for(int64_t n, int per) { return static_cast<int>((n + per - 1) / per); }

int key_bits(int64_t rows) {
  int bits = 0;
  const uint64_t maxkey = rows > 0 ? static_cast<uint64_t>(rows - 1) : 0;
  while (bits < 32 && (maxkey >> bits) != 0) ++bits;
  return bits;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

GradWorkspace plan_grad_workspace(const el_tables& tab, int64_t n, void* base) {
  GradWorkspace ws;
  ws.n = n;
  if (n <= 0) return ws;
  const int F = tab.num_tables, D = tab.dim;
  // local rows: below the largest table's rows (below all rows when that is not known)
  const int bits = key_bits(tab.max_rows > 0 ? tab.max_rows : tab.total_rows);
  // the fewest passes of <= kRadixBits, at least one (the first pass writes the keys)
  ws.passes = bits > 0 ? (bits + kRadixBits - 1) / kRadixBits : 1;
  ws.rbits = bits > 0 ? (bits + ws.passes - 1) / ws.passes : 1;  // equal widths
  // tiles: every table's last tile may be short, so at most ceil(n / tile) + F of them
  ws.nblocks = (n + kSortTile - 1) / kSortTile + F;
  ws.nranges = (n + kMinRange - 1) / kMinRange;
  const int64_t m_hist = ws.nblocks * (int64_t{1} << ws.rbits);
  const int64_t scan_len = n;
  char* p = static_cast<char*>(base);
  size_t off = 0;
  auto take = [&](size_t bytes) -> void* {
    void* r = p ? p + off : nullptr;
    off += align256(bytes);
    return r;
  };
  ws.keys0 = static_cast<uint32_t*>(take(4 * n));
  ws.vals0 = static_cast<uint32_t*>(take(4 * n));
  ws.keys1 = static_cast<uint32_t*>(take(4 * n));
  ws.vals1 = static_cast<uint32_t*>(take(4 * n));
  ws.tile_prefix = static_cast<int32_t*>(take(4 * (static_cast<size_t>(F) + 1)));
  ws.tiles = static_cast<SortTile*>(take(sizeof(SortTile) * ws.nblocks));
  ws.hist = static_cast<uint32_t*>(take(4 * m_hist));
  ws.hist_scan = static_cast<uint32_t*>(take(4 * m_hist));
  ws.dtotal = static_cast<uint32_t*>(take(4 << kRadixBits));
  ws.flags = static_cast<uint32_t*>(take(4 * n));
  ws.flags_scan = static_cast<uint32_t*>(take(4 * n));
  int64_t len = scan_len;
  for (int l = 0; l < 4; ++l) {
    len = (len + kScanTile - 1) / kScanTile;
    ws.scan_level[l][0] = static_cast<uint32_t*>(take(4 * len));
    ws.scan_level[l][1] = static_cast<uint32_t*>(take(4 * len));
    if (len <= 1) break;
  }
  ws.range_head = static_cast<float*>(take(sizeof(float) * ws.nranges * D));
  ws.range_tail = static_cast<float*>(take(sizeof(float) * ws.nranges * D));
  ws.range_flags = static_cast<uint32_t*>(take(4 * ws.nranges));
  ws.bytes = off;
  return ws;
}

el_status launch_exclusive_scan(const uint32_t* in, uint32_t* out, int64_t n,
                                uint32_t* const level[4][2], hipStream_t stream) {
  if (n <= 0) return EL_OK;
  const int tiles = blocks_for(n, kScanTile);
  hipLaunchKernelGGL(k_scan_tile, dim3(tiles), dim3(256), 0, stream, in, out, n, level[0][0]);
  el_status st = check_launch("scan");
  if (st != EL_OK || tiles == 1) return st;
  st = launch_exclusive_scan(level[0][0], level[0][1], tiles, level + 1, stream);
  if (st != EL_OK) return st;
  hipLaunchKernelGGL(k_scan_add, dim3(blocks_for(n, 256)), dim3(256), 0, stream, out, n,
                     static_cast<const uint32_t*>(level[0][1]));
  return check_launch("scan");
}

namespace {

template <int RB>
el_status radix_pass_t(const el_tables& tab, const el_bags& bags, bool hash, const GradWorkspace& ws,
                       int pass, const uint32_t* kin, const uint32_t* vin, uint32_t* kout, uint32_t* vout,
                       hipStream_t stream) {
  const int nb = static_cast<int>(ws.nblocks);
  const int shift = pass * ws.rbits;
  const bool first = pass == 0;
  const int last = pass == ws.passes - 1 ? 1 : 0;
  if (first)
    hipLaunchKernelGGL((k_radix_hist<RB, true>), dim3(nb), dim3(256), 0, stream, kin, bags.indices,
                       static_cast<const SortTile*>(ws.tiles), tab.row_offset, hash ? 1 : 0, shift, ws.hist, nb);
  else
    hipLaunchKernelGGL((k_radix_hist<RB, false>), dim3(nb), dim3(256), 0, stream, kin, bags.indices,
                       static_cast<const SortTile*>(ws.tiles), tab.row_offset, hash ? 1 : 0, shift, ws.hist, nb);
  el_status st = check_launch("radix_hist");
  if (st != EL_OK) return st;
  hipLaunchKernelGGL(k_digit_scan, dim3(1 << RB), dim3(256), 0, stream,
                     static_cast<const uint32_t*>(ws.hist), ws.hist_scan, nb, ws.dtotal);
  if ((st = check_launch("radix_scan")) != EL_OK) return st;
  if (first)
    hipLaunchKernelGGL((k_radix_scatter<RB, true>), dim3(round_up8(nb)), dim3(256), 0, stream, kin, bags.indices, vin,
                       static_cast<const SortTile*>(ws.tiles), tab.row_offset, hash ? 1 : 0, last, shift,
                       static_cast<const uint32_t*>(ws.hist_scan), static_cast<const uint32_t*>(ws.dtotal),
                       kout, vout, nb);
  else
    hipLaunchKernelGGL((k_radix_scatter<RB, false>), dim3(round_up8(nb)), dim3(256), 0, stream, kin, bags.indices, vin,
                       static_cast<const SortTile*>(ws.tiles), tab.row_offset, hash ? 1 : 0, last, shift,
                       static_cast<const uint32_t*>(ws.hist_scan), static_cast<const uint32_t*>(ws.dtotal),
                       kout, vout, nb);
  return check_launch("radix_scatter");
}

el_status radix_pass(const el_tables& tab, const el_bags& bags, bool hash, const GradWorkspace& ws, int pass,
                     const uint32_t* kin, const uint32_t* vin, uint32_t* kout, uint32_t* vout,
                     hipStream_t stream) {
  switch (ws.rbits) {
    case 1: return radix_pass_t<1>(tab, bags, hash, ws, pass, kin, vin, kout, vout, stream);
    case 2: return radix_pass_t<2>(tab, bags, hash, ws, pass, kin, vin, kout, vout, stream);
    case 3: return radix_pass_t<3>(tab, bags, hash, ws, pass, kin, vin, kout, vout, stream);
    case 4: return radix_pass_t<4>(tab, bags, hash, ws, pass, kin, vin, kout, vout, stream);
    case 5: return radix_pass_t<5>(tab, bags, hash, ws, pass, kin, vin, kout, vout, stream);
    case 6: return radix_pass_t<6>(tab, bags, hash, ws, pass, kin, vin, kout, vout, stream);
    case 7: return radix_pass_t<7>(tab, bags, hash, ws, pass, kin, vin, kout, vout, stream);
    case 8: return radix_pass_t<8>(tab, bags, hash, ws, pass, kin, vin, kout, vout, stream);
    case 9: return radix_pass_t<9>(tab, bags, hash, ws, pass, kin, vin, kout, vout, stream);
  }
  return set_error(EL_ERR_UNSUPPORTED, "radix digit width out of range");
}

}  // namespace

el_status launch_grad_sort_core(const el_tables& tab, const el_bags& bags, uint32_t flags,
                                GradWorkspace& ws, uint32_t** sorted_keys, uint32_t** sorted_vals,
                                hipStream_t stream) {
  const int64_t nbags = static_cast<int64_t>(tab.num_tables) * bags.batch;
  const int nb = static_cast<int>(ws.nblocks);
  hipLaunchKernelGGL(k_sort_tiles, dim3(1), dim3(256), 0, stream, bags.offsets, bags.batch,
                     tab.num_tables, ws.tile_prefix);
  el_status st = check_launch("sort_tiles");
  if (st != EL_OK) return st;
  hipLaunchKernelGGL(k_tile_info, dim3(blocks_for(nb, 256)), dim3(256), 0, stream, bags.offsets, bags.batch,
                     tab.num_tables, static_cast<const int32_t*>(ws.tile_prefix), nb, ws.tiles);
  if ((st = check_launch("tile_info")) != EL_OK) return st;
  hipLaunchKernelGGL(k_build_vals, dim3(blocks_for(nbags, 256)), dim3(256), 0, stream, bags.offsets,
                     static_cast<int32_t>(nbags), ws.vals0);
  if ((st = check_launch("build_vals")) != EL_OK) return st;
  // pass 0 reads the indices and vals0; then the buffers alternate, pass p writing
  // keys1 / vals1 when p is even
  const bool hash = (flags & EL_FLAG_HASH_INDICES) != 0;
  const uint32_t *kin = ws.keys0, *vin = ws.vals0;
  for (int pass = 0; pass < ws.passes; ++pass) {
    uint32_t* kout = pass % 2 == 0 ? ws.keys1 : ws.keys0;
    uint32_t* vout = pass % 2 == 0 ? ws.vals1 : ws.vals0;
    if ((st = radix_pass(tab, bags, hash, ws, pass, kin, vin, kout, vout, stream)) != EL_OK) return st;
    kin = kout;
    vin = vout;
  }
  sorted_buffers(ws, sorted_keys, sorted_vals);
  return EL_OK;
}

void sorted_buffers(const GradWorkspace& ws, uint32_t** sorted_keys, uint32_t** sorted_vals) {
  const bool odd = ws.passes % 2 != 0;  // every pass swaps the buffers
  *sorted_keys = odd ? ws.keys1 : ws.keys0;
  *sorted_vals = odd ? ws.vals1 : ws.vals0;
}

el_status launch_segments(const GradWorkspace& ws, const uint32_t* sorted_keys,
                          uint32_t* unique_rows, uint32_t* seg_offsets, uint32_t* num_unique,
                          hipStream_t stream) {
  if (ws.n <= 0) {
    hipLaunchKernelGGL(k_seg_empty, dim3(1), dim3(64), 0, stream, seg_offsets, num_unique);
    return check_launch("segments");
  }
  const int nb = blocks_for(ws.n, 256);
  hipLaunchKernelGGL(k_seg_flags, dim3(nb), dim3(256), 0, stream, sorted_keys, ws.n, ws.flags);
  el_status st = check_launch("segments");
  if (st != EL_OK) return st;
  if ((st = launch_exclusive_scan(ws.flags, ws.flags_scan, ws.n, ws.scan_level, stream)) != EL_OK)
    return st;
  hipLaunchKernelGGL(k_seg_emit, dim3(nb), dim3(256), 0, stream, sorted_keys,
                     static_cast<const uint32_t*>(ws.flags), static_cast<const uint32_t*>(ws.flags_scan),
                     ws.n, unique_rows, seg_offsets, num_unique);
  return check_launch("segments");
}

}  // namespace el
