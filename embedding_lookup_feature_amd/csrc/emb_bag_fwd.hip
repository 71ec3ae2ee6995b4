// emb_bag_fwd.hip -- embedding-bag gather with sum pooling over CSR bags (gfx950).
//
// Page "DLRM For PyTorch", §Model architecture: one embedding table per categorical
// feature; the embedding vector of a sample for a table is here the sum of the rows its
// bag names (hotness 1 = one row).  Bags are table-major (bag g = t*B + b).
//
// Mapping.  A launch covers the samples [b0, b0 + Bc) (all of them for emb_bag_fwd); its
// bags are numbered table-major within that range.  A wavefront gathers NB = NG * U
// consecutive bags in one pass and exits: the wave is cut into NG groups of L lanes
// (L = row bytes / 16, rounded up to a power of two; a group covers one row with 16-byte
// loads) and every group pools U bags.
//   1. lane i < NB loads the CSR bounds of bag i and the first row of its table
//      (independent loads, one round trip), then the bag's first index;
//   2. every group issues the first-row loads of its U bags back to back, so U row loads
//      per lane are in flight (for hotness-1 bags this is the whole gather); later entries
//      of multi-hot bags follow in ascending CSR order, 4 loads in flight;
//   3. all NB pooled rows are stored at the end, pooled vector (b, t) at element
//      b * ostride + ocol + t * D of the output (the [B][F][D] array: ostride = F*D,
//      ocol = 0; the cat interaction's output rows: ostride = out_stride, ocol = D).
// A wave never waits for its own stores (on this architecture loads and stores share one
// completion counter), and a new wave takes its slot as soon as it is done.
//
// Long bags (on average four lookups or more, rows of at least 128 bytes): k_emb_bag_long
// gives each group one bag, so a wave's NG bags advance side by side instead of a group's
// U bags one after another.  A group walks its bag in rounds of R = 8 entries: the first R
// lanes of the group hold the round's indices (loaded one round ahead, while the rows of the
// current round are in flight), and the group issues the round's R row loads before adding
// any of them, in CSR order.  The sum starts from -0.0, which leaves the first row unchanged
// bit for bit (x + (-0) = x for every x, signed zeros included), so the result is the same
// as starting from the first row; an empty bag stores +0.  Sums are fp32
// in CSR order and rounded once to the output type, so a hotness-1 gather returns the row
// itself (bit-exact up to the output rounding).
#include "el_internal.hpp"

namespace el {
namespace {

template <int L, int NVL>
constexpr int bags_per_group() {
  constexpr int NG = 64 / L;
  constexpr int byreg = 16 / NVL;  // keep U * NVL 16-byte vectors <= 16 per lane
  constexpr int u = 64 / NG < 8 ? 64 / NG : 8;
  return u < byreg ? u : byreg;
}

template <class TT, class OT, int L, int NVL>
__global__ __launch_bounds__(256) void k_emb_bag_fwd(
    const typename TT::S* __restrict__ W, const int64_t* __restrict__ row_off,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ off, int32_t B, int32_t F,
    int32_t D, int32_t nvec, uint32_t hash, typename OT::S* __restrict__ out, int64_t ostride,
    int32_t ocol, int32_t nbags, int32_t b0, int32_t Bc) {
  constexpr int E = epv<TT>();
  constexpr int NG = 64 / L;                  // bag groups per wave
  constexpr int U = bags_per_group<L, NVL>();  // bags per group
  constexpr int NB = NG * U;                  // bags per wave

  const int lane = threadIdx.x & 63;
  const int grp = lane / L;
  const int gl = lane % L;
  const int blk = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t g0l = (static_cast<int64_t>(blk) * 4 + (threadIdx.x >> 6)) * NB;
  if (g0l >= nbags) return;
  const int g0 = static_cast<int>(g0l);  // < nbags < 2^31

  // 1. per-lane bag metadata (lanes < NB): bounds, table, table base; then the first index
  int s = 0, e = 0, r0 = 0, t = -1, b = 0, nt = 1;
  int64_t base = 0;
  if (lane < NB && g0l + lane < nbags) {
    const int gc = g0 + lane;  // bag of the launch: table t, sample b0 + (gc - t * Bc)
    t = gc / Bc;
    b = b0 + (gc - t * Bc);
    const int g = t * B + b;
    // plain loads: neighbouring wavefronts read the same lines of bounds and indices
    s = off[g];
    e = off[g + 1];
    base = row_off[t];
    if (hash) nt = static_cast<int32_t>(row_off[t + 1] - base);
  }
  if (e > s) {
    r0 = idx[s];
    if (hash) r0 = floor_mod(r0, nt);
  }

  // 2. first rows of the group's U bags, all in flight together
  uint4 v[U][NVL];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int bi = u * NG + grp;
    const int bs = __shfl(s, bi), be = __shfl(e, bi), r = __shfl(r0, bi);
    const int64_t bse = __shfl(base, bi);
    const typename TT::S* row = W + (bse + r) * D;
#pragma unroll
    for (int m = 0; m < NVL; ++m) {
      v[u][m] = uint4{0, 0, 0, 0};
      const int c = gl + m * L;
      if (be > bs && c < nvec) v[u][m] = load16<TT>(row + c * E);
    }
  }
  float acc[U][NVL][E];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int m = 0; m < NVL; ++m) unpack16<TT>(v[u][m], acc[u][m]);

  //    further entries of multi-hot bags, in CSR order
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int bi = u * NG + grp;
    const int bs = __shfl(s, bi), be = __shfl(e, bi), ntb = __shfl(nt, bi);
    const int64_t bse = __shfl(base, bi);
    for (int k = bs + 1; k < be; k += 4) {
      // indices and rows of the next 4 entries, all loads issued before any is used
      // (entries past the bag end re-read its last entry and are not added)
      int r[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        r[q] = idx[k + q < be ? k + q : be - 1];
        if (hash) r[q] = floor_mod(r[q], ntb);
      }
      uint4 w[4][NVL];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const typename TT::S* row = W + (bse + r[q]) * D;
#pragma unroll
        for (int m = 0; m < NVL; ++m) {
          const int c = gl + m * L;
          w[q][m] = load16<TT>(row + (c < nvec ? c : nvec - 1) * E);
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (k + q < be) {
#pragma unroll
          for (int m = 0; m < NVL; ++m) {
            float f[E];
            unpack16<TT>(w[q][m], f);
#pragma unroll
            for (int x = 0; x < E; ++x) acc[u][m][x] += f[x];
          }
        }
      }
    }
  }

  // 3. store every pooled row
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int bi = u * NG + grp;
    const int tb = __shfl(t, bi), bb = __shfl(b, bi);
    if (tb >= 0) {
      typename OT::S* dst = out + static_cast<int64_t>(bb) * ostride + ocol + static_cast<int64_t>(tb) * D;
#pragma unroll
      for (int m = 0; m < NVL; ++m) {
        const int c = gl + m * L;
        if (c < nvec) store_n<OT, E>(dst + c * E, acc[u][m]);
      }
    }
  }
}

template <class TT, class OT, int L, int NVL>
__global__ __launch_bounds__(256) void k_emb_bag_long(
    const typename TT::S* __restrict__ W, const int64_t* __restrict__ row_off,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ off, int32_t B, int32_t D,
    int32_t nvec, uint32_t hash, typename OT::S* __restrict__ out, int64_t ostride, int32_t ocol,
    int32_t nbags, int32_t b0, int32_t Bc) {
  constexpr int E = epv<TT>();
  constexpr int NG = 64 / L;  // bags per wave, one per group
  constexpr int R = 8;        // entries per round
  static_assert(L >= R, "the round's indices sit in the group's first R lanes");
  const int lane = threadIdx.x & 63;
  const int grp = lane / L;
  const int gl = lane % L;
  const int blk = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t gw = (static_cast<int64_t>(blk) * 4 + (threadIdx.x >> 6)) * NG;
  if (gw >= nbags) return;  // the whole wave
  const int64_t gc = gw + grp;
  const bool valid = gc < nbags;  // group-uniform
  int s = 0, e = 0, t = 0, b = 0, nt = 1;
  int64_t base = 0;
  if (valid) {
    t = static_cast<int>(gc / Bc);
    b = b0 + static_cast<int>(gc - static_cast<int64_t>(t) * Bc);
    const int64_t g = static_cast<int64_t>(t) * B + b;
    // plain loads: neighbouring wavefronts read the same lines of bounds and indices
    s = off[g];
    e = off[g + 1];
    base = row_off[t];
    if (hash) nt = static_cast<int32_t>(row_off[t + 1] - base);
  }
  float acc[NVL][E];
#pragma unroll
  for (int m = 0; m < NVL; ++m)
#pragma unroll
    for (int x = 0; x < E; ++x) acc[m][x] = -0.0f;
  const int src0 = grp * L;  // the group's first lane
  int ri = 0;
  if (s + (gl & (R - 1)) < e) {  // (a table without rows has only empty bags)
    ri = idx[s + (gl & (R - 1))];
    if (hash) ri = floor_mod(ri, nt);
  }
  for (int k = s; k < e; k += R) {  // group-uniform trip count
    // the next round's indices, in flight with this round's rows
    const int kn = k + R + (gl & (R - 1));
    int rn = kn < e ? idx[kn] : 0;
    uint4 w[R][NVL];
#pragma unroll
    for (int q = 0; q < R; ++q) {
      const int rq = __shfl(ri, src0 + q);  // entries past the end read row 0, never added
      const typename TT::S* row = W + (base + rq) * D;
#pragma unroll
      for (int m = 0; m < NVL; ++m) {
        const int c = gl + m * L;
        w[q][m] = load16<TT>(row + (c < nvec ? c : nvec - 1) * E);
      }
    }
#pragma unroll
    for (int q = 0; q < R; ++q) {
      if (k + q < e) {
#pragma unroll
        for (int m = 0; m < NVL; ++m) {
          float f[E];
          unpack16<TT>(w[q][m], f);
#pragma unroll
          for (int x = 0; x < E; ++x) acc[m][x] += f[x];
        }
      }
    }
    if (hash) rn = floor_mod(rn, nt);
    ri = rn;
  }
  if (!valid) return;
  if (e <= s) {  // an empty bag pools to +0
#pragma unroll
    for (int m = 0; m < NVL; ++m)
#pragma unroll
      for (int x = 0; x < E; ++x) acc[m][x] = 0.0f;
  }
  typename OT::S* dst = out + static_cast<int64_t>(b) * ostride + ocol + static_cast<int64_t>(t) * D;
#pragma unroll
  for (int m = 0; m < NVL; ++m) {
    const int c = gl + m * L;
    if (c < nvec) store_n<OT, E>(dst + c * E, acc[m]);
  }
}

template <class TT, class OT, int L, int NVL>
el_status launch_t(const el_tables& tab, const el_bags& bags, uint32_t flags, void* out,
                   int64_t ostride, int ocol, int nvec, int b0, int Bc, hipStream_t stream) {
  const int64_t nbags = static_cast<int64_t>(tab.num_tables) * Bc;
  if constexpr (L >= 8) {
    // long bags: one bag per group (four lookups or more per bag on average)
    if (bags.nnz >= 4 * static_cast<int64_t>(tab.num_tables) * bags.batch) {
      const int64_t waves = (nbags + (64 / L) - 1) / (64 / L);
      const int blocks = round_up8((waves + 3) / 4);
      hipLaunchKernelGGL((k_emb_bag_long<TT, OT, L, NVL>), dim3(blocks), dim3(256), 0, stream,
                         static_cast<const typename TT::S*>(tab.base), tab.row_offset, bags.indices,
                         bags.offsets, bags.batch, tab.dim, nvec, (flags & EL_FLAG_HASH_INDICES) ? 1u : 0u,
                         static_cast<typename OT::S*>(out), ostride, ocol, static_cast<int32_t>(nbags), b0, Bc);
      return check_launch("emb_bag_fwd");
    }
  }
  constexpr int NB = (64 / L) * bags_per_group<L, NVL>();
  const int64_t waves = (nbags + NB - 1) / NB;
  const int blocks = round_up8((waves + 3) / 4);
  hipLaunchKernelGGL((k_emb_bag_fwd<TT, OT, L, NVL>), dim3(blocks), dim3(256), 0, stream,
                     static_cast<const typename TT::S*>(tab.base), tab.row_offset, bags.indices,
                     bags.offsets, bags.batch, tab.num_tables, tab.dim, nvec,
                     (flags & EL_FLAG_HASH_INDICES) ? 1u : 0u,
                     static_cast<typename OT::S*>(out), ostride, ocol, static_cast<int32_t>(nbags), b0, Bc);
  return check_launch("emb_bag_fwd");
}

template <class TT, class OT>
el_status dispatch_shape(const el_tables& tab, const el_bags& bags, uint32_t flags, void* out,
                         int64_t ostride, int ocol, int b0, int Bc, hipStream_t stream) {
  const int nvec = static_cast<int>(tab.dim * sizeof(typename TT::S) / 16);
  if (nvec <= 1) return launch_t<TT, OT, 1, 1>(tab, bags, flags, out, ostride, ocol, nvec, b0, Bc, stream);
  if (nvec <= 2) return launch_t<TT, OT, 2, 1>(tab, bags, flags, out, ostride, ocol, nvec, b0, Bc, stream);
  if (nvec <= 4) return launch_t<TT, OT, 4, 1>(tab, bags, flags, out, ostride, ocol, nvec, b0, Bc, stream);
  if (nvec <= 8) return launch_t<TT, OT, 8, 1>(tab, bags, flags, out, ostride, ocol, nvec, b0, Bc, stream);
  if (nvec <= 16) return launch_t<TT, OT, 16, 1>(tab, bags, flags, out, ostride, ocol, nvec, b0, Bc, stream);
  if (nvec <= 32) return launch_t<TT, OT, 32, 1>(tab, bags, flags, out, ostride, ocol, nvec, b0, Bc, stream);
  if (nvec <= 64) return launch_t<TT, OT, 64, 1>(tab, bags, flags, out, ostride, ocol, nvec, b0, Bc, stream);
  if (nvec <= 128) return launch_t<TT, OT, 64, 2>(tab, bags, flags, out, ostride, ocol, nvec, b0, Bc, stream);
  if (nvec <= 256) return launch_t<TT, OT, 64, 4>(tab, bags, flags, out, ostride, ocol, nvec, b0, Bc, stream);
  return set_error(EL_ERR_UNSUPPORTED, "emb_bag_fwd: rows longer than 4096 bytes are not supported");
}

template <class TT>
el_status dispatch_out(const el_tables& tab, const el_bags& bags, uint32_t flags, void* out,
                       el_dtype out_dtype, int64_t ostride, int ocol, int b0, int Bc,
                       hipStream_t stream) {
  switch (out_dtype) {
    case EL_F32: return dispatch_shape<TT, F32T>(tab, bags, flags, out, ostride, ocol, b0, Bc, stream);
    case EL_F16: return dispatch_shape<TT, F16T>(tab, bags, flags, out, ostride, ocol, b0, Bc, stream);
    case EL_BF16: return dispatch_shape<TT, BF16T>(tab, bags, flags, out, ostride, ocol, b0, Bc, stream);
    default: break;
  }
  return set_error(EL_ERR_INVALID_ARG, "emb_bag_fwd: unknown output dtype");
}

}  // namespace

el_status launch_emb_bag_fwd(const el_tables& tab, const el_bags& bags, uint32_t flags, void* out,
                             el_dtype out_dtype, hipStream_t stream, int b0, int Bc,
                             int64_t ostride, int ocol) {
  if (Bc < 0) Bc = bags.batch;
  if (ostride < 0) ostride = static_cast<int64_t>(tab.num_tables) * tab.dim;
  switch (tab.dtype) {
    case EL_F32: return dispatch_out<F32T>(tab, bags, flags, out, out_dtype, ostride, ocol, b0, Bc, stream);
    case EL_F16: return dispatch_out<F16T>(tab, bags, flags, out, out_dtype, ostride, ocol, b0, Bc, stream);
    case EL_BF16: return dispatch_out<BF16T>(tab, bags, flags, out, out_dtype, ostride, ocol, b0, Bc, stream);
    default: break;
  }
  return set_error(EL_ERR_INVALID_ARG, "emb_bag_fwd: unknown table dtype");
}

}  // namespace el
