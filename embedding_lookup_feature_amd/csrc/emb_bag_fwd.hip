// emb_bag_fwd.hip -- embedding-bag gather with sum pooling over CSR bags (gfx950).
//
// Page "DLRM For PyTorch", §Model architecture: one embedding table per categorical
// feature; the embedding vector of a sample for a table is here the sum of the rows its
// bag names (hotness 1 = one row).  Bags are table-major (bag g = t*B + b).
//
// Mapping.  A wavefront owns a batch of 64 consecutive bags.  Lane i first streams in the
// CSR bounds of bag i and its first index with non-temporal loads (coalesced, read once).
// The wave is cut into groups of L lanes; a group covers one table row with 16-byte
// loads (L = row bytes / 16, rounded up to a power of two).  The groups then walk the 64
// bags in rounds; U rounds are issued back to back so that U independent row loads per
// lane are in flight before the first is consumed (for hotness-1 bags this is the whole
// gather).  Further entries of a bag follow in ascending CSR order, 4 loads in flight.
// Sums are fp32 in CSR order and rounded once to the output type, so a hotness-1 gather
// returns the row itself (bit-exact copy up to the output rounding).
#include "el_internal.hpp"

namespace el {
namespace {

template <class TT, class OT, int L, int NVL>
__global__ __launch_bounds__(256) void k_emb_bag_fwd(
    const typename TT::S* __restrict__ W, const int64_t* __restrict__ row_off,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ off, int32_t B, int32_t F,
    int32_t D, int32_t nvec, uint32_t hash, typename OT::S* __restrict__ out, int32_t nbags) {
  constexpr int E = epv<TT>();
  constexpr int NG = 64 / L;  // bag groups per wave
  constexpr int R = 64 / NG;  // rounds to cover the wave's 64 bags
  constexpr int U0 = 8 / NVL;
  constexpr int U = R < U0 ? R : U0;  // rounds issued together

  const int lane = threadIdx.x & 63;
  const int grp = lane / L;
  const int gl = lane % L;
  const int blk = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t g0l = (static_cast<int64_t>(blk) * 4 + (threadIdx.x >> 6)) * 64;
  if (g0l >= nbags) return;
  const int g0 = static_cast<int>(g0l);  // < nbags < 2^31

  int s = 0, e = 0, r0 = 0;
  if (g0l + lane < nbags) {
    s = ld_stream(off + g0 + lane);
    e = ld_stream(off + g0 + lane + 1);
    if (e > s) r0 = ld_stream(idx + s);
  }

  for (int j0 = 0; j0 < R; j0 += U) {
    uint4 v[U][NVL];
    int bs[U], be[U], tt[U], bb[U], nt[U];
    int64_t base[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int bi = (j0 + u) * NG + grp;
      bs[u] = __shfl(s, bi);
      be[u] = __shfl(e, bi);
      int r = __shfl(r0, bi);
      const bool ok = g0l + bi < nbags;
      const int g = ok ? g0 + bi : 0;
      const int t = ok ? g / B : 0;
      tt[u] = ok ? t : -1;
      bb[u] = g - t * B;
      base[u] = ok ? row_off[t] : 0;
      nt[u] = (ok && hash) ? static_cast<int32_t>(row_off[t + 1] - base[u]) : 1;
      const bool has = ok && be[u] > bs[u];
      if (hash) r = floor_mod(r, nt[u]);
      const typename TT::S* row = W + (base[u] + r) * D;
#pragma unroll
      for (int m = 0; m < NVL; ++m) {
        const int c = gl + m * L;
        v[u][m] = (has && c < nvec) ? load16<TT>(row + c * E) : uint4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (tt[u] < 0) continue;
      float acc[NVL][E];
#pragma unroll
      for (int m = 0; m < NVL; ++m) unpack16<TT>(v[u][m], acc[m]);
      for (int k = bs[u] + 1; k < be[u]; k += 4) {
        uint4 w[4][NVL];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (k + q < be[u]) {
            int r = idx[k + q];
            if (hash) r = floor_mod(r, nt[u]);
            const typename TT::S* row = W + (base[u] + r) * D;
#pragma unroll
            for (int m = 0; m < NVL; ++m) {
              const int c = gl + m * L;
              w[q][m] = c < nvec ? load16<TT>(row + c * E) : uint4{0, 0, 0, 0};
            }
          }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (k + q < be[u]) {
#pragma unroll
            for (int m = 0; m < NVL; ++m) {
              float f[E];
              unpack16<TT>(w[q][m], f);
#pragma unroll
              for (int x = 0; x < E; ++x) acc[m][x] += f[x];
            }
          }
        }
      }
      typename OT::S* dst = out + (static_cast<int64_t>(bb[u]) * F + tt[u]) * D;
#pragma unroll
      for (int m = 0; m < NVL; ++m) {
        const int c = gl + m * L;
        if (c < nvec) store_n<OT, E>(dst + c * E, acc[m]);
      }
    }
  }
}

template <class TT, class OT, int L, int NVL>
el_status launch_t(const el_tables& tab, const el_bags& bags, uint32_t flags, void* out,
                   int nvec, hipStream_t stream) {
  const int64_t nbags = static_cast<int64_t>(tab.num_tables) * bags.batch;
  const int64_t waves = (nbags + 63) / 64;
  const int blocks = round_up8((waves + 3) / 4);
  hipLaunchKernelGGL((k_emb_bag_fwd<TT, OT, L, NVL>), dim3(blocks), dim3(256), 0, stream,
                     static_cast<const typename TT::S*>(tab.base), tab.row_offset, bags.indices,
                     bags.offsets, bags.batch, tab.num_tables, tab.dim, nvec,
                     (flags & EL_FLAG_HASH_INDICES) ? 1u : 0u,
                     static_cast<typename OT::S*>(out), static_cast<int32_t>(nbags));
  return check_launch("emb_bag_fwd");
}

template <class TT, class OT>
el_status dispatch_shape(const el_tables& tab, const el_bags& bags, uint32_t flags, void* out,
                         hipStream_t stream) {
  const int nvec = static_cast<int>(tab.dim * sizeof(typename TT::S) / 16);
  if (nvec <= 1) return launch_t<TT, OT, 1, 1>(tab, bags, flags, out, nvec, stream);
  if (nvec <= 2) return launch_t<TT, OT, 2, 1>(tab, bags, flags, out, nvec, stream);
  if (nvec <= 4) return launch_t<TT, OT, 4, 1>(tab, bags, flags, out, nvec, stream);
  if (nvec <= 8) return launch_t<TT, OT, 8, 1>(tab, bags, flags, out, nvec, stream);
  if (nvec <= 16) return launch_t<TT, OT, 16, 1>(tab, bags, flags, out, nvec, stream);
  if (nvec <= 32) return launch_t<TT, OT, 32, 1>(tab, bags, flags, out, nvec, stream);
  if (nvec <= 64) return launch_t<TT, OT, 64, 1>(tab, bags, flags, out, nvec, stream);
  if (nvec <= 128) return launch_t<TT, OT, 64, 2>(tab, bags, flags, out, nvec, stream);
  if (nvec <= 256) return launch_t<TT, OT, 64, 4>(tab, bags, flags, out, nvec, stream);
  return set_error(EL_ERR_UNSUPPORTED, "emb_bag_fwd: rows longer than 4096 bytes are not supported");
}

template <class TT>
el_status dispatch_out(const el_tables& tab, const el_bags& bags, uint32_t flags, void* out,
                       el_dtype out_dtype, hipStream_t stream) {
  switch (out_dtype) {
    case EL_F32: return dispatch_shape<TT, F32T>(tab, bags, flags, out, stream);
    case EL_F16: return dispatch_shape<TT, F16T>(tab, bags, flags, out, stream);
    case EL_BF16: return dispatch_shape<TT, BF16T>(tab, bags, flags, out, stream);
  }
  return set_error(EL_ERR_INVALID_ARG, "emb_bag_fwd: unknown output dtype");
}

}  // namespace

el_status launch_emb_bag_fwd(const el_tables& tab, const el_bags& bags, uint32_t flags, void* out,
                             el_dtype out_dtype, hipStream_t stream) {
  switch (tab.dtype) {
    case EL_F32: return dispatch_out<F32T>(tab, bags, flags, out, out_dtype, stream);
    case EL_F16: return dispatch_out<F16T>(tab, bags, flags, out, out_dtype, stream);
    case EL_BF16: return dispatch_out<BF16T>(tab, bags, flags, out, out_dtype, stream);
  }
  return set_error(EL_ERR_INVALID_ARG, "emb_bag_fwd: unknown table dtype");
}

}  // namespace el
