// emb_dot_fwd.hip -- the embedding-bag gather fused with the dot-interaction forward
// (gfx950).
//
// Page "DLRM For PyTorch", §Model architecture: the pooled embedding vectors of a sample
// (one per table) and the bottom-MLP output x0 feed the dot interaction.  Computed apart,
// the pooled vectors make a round trip through HBM (written by the gather, read back by
// the interaction).  Here one wavefront builds a sample's V x D tile straight in LDS: it
// gathers the sample's table rows, sums each bag in fp32 in CSR order, rounds once to the
// activation type (exactly as emb_bag_fwd does) and writes the rounded vectors to the LDS
// tile; the Gram products then run on the tile exactly as in dot_interact_fwd.  Results are
// bit-identical to the two separate calls.
// Gathering sample by sample touches every table at once and so loses the L2 locality of
// the table-major gather; the fused kernel is therefore used only when the pooled vectors
// are not stored (inference), and emb_dot_fwd with emb_out runs the two kernels on chunks of
// samples instead (launch_emb_dot_fwd).
//
// Pipeline per wavefront (grid-strided over samples j, j+G, ...): while sample j is
// reduced and multiplied, the rows of sample j+G, the first indices of sample j+2G and the
// CSR bounds of sample j+3G are in flight.  Every load is issued unconditionally (sample
// numbers past the end are clamped), every store count is fixed and each trip issues its
// loads before its stores, so waiting for a load never waits for a store (loads and stores
// share one in-order completion counter).
#include <algorithm>

#include "el_internal.hpp"
#include "el_mfma.hpp"

namespace el {
namespace {

// 8 consecutive elements of a table row: 32 bytes (fp32) or 16 bytes (16-bit).
template <class TT>
struct Unit {
  static constexpr int NV = static_cast<int>(sizeof(typename TT::S)) / 2;  // 16-byte vectors
  u32x4 v[NV];
};

template <class TT>
__device__ inline void load_unit(Unit<TT>& u, const typename TT::S* p) {
#pragma unroll
  for (int i = 0; i < Unit<TT>::NV; ++i) u.v[i] = reinterpret_cast<const u32x4*>(p)[i];
}

template <class TT>
__device__ inline void unit_to_f(const Unit<TT>& u, float* f) {
#pragma unroll
  for (int i = 0; i < Unit<TT>::NV; ++i) {
    const uint4 w = {u.v[i][0], u.v[i][1], u.v[i][2], u.v[i][3]};
    unpack16<TT>(w, f + i * epv<TT>());
  }
}

// An empty register use: the compiler waits here for the load that produced `v`.
template <class T>
__device__ inline void settle(const T& v) {
  asm volatile("" ::"v"(v));
}

// 8 floats -> 8 x 16-bit of IT (round to nearest even), packed as 16 bytes.
template <class IT>
__device__ inline u32x4 pack8(const float* f) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r[i] = static_cast<uint32_t>(IT::from_f(f[2 * i])) | (static_cast<uint32_t>(IT::from_f(f[2 * i + 1])) << 16);
  return r;
}

// TT: table type; IT: activation type (16-bit: pooled vectors, x0 and out); NU: row units
// (8 elements) per lane; SPL: 16-byte output-row chunks per lane.
template <class TT, class IT, int NU, int SPL>
__global__ __launch_bounds__(64) void k_emb_dot_fwd(
    const typename TT::S* __restrict__ W, const int64_t* __restrict__ row_off,
    const int32_t* __restrict__ idx, int32_t nnz, const int32_t* __restrict__ off, int32_t B,
    int32_t F, int32_t D, uint32_t hash, const uint16_t* __restrict__ x0,
    uint16_t* __restrict__ out, int32_t out_stride) {
  extern __shared__ uint4 smem[];
  char* lds = reinterpret_cast<char*>(smem);
  const int lane = threadIdx.x;
  const int V = F + 1;
  const int P = V * (V - 1) / 2;
  const int pitch = D * 2 + 16;
  const int obase = V * pitch;
  const int obytes = (out_stride * 2 + 15) / 16 * 16;
  const int trash = obase + obytes;
  uint16_t* ostage = reinterpret_cast<uint16_t*>(lds + obase);
  const int nur = D / 8;       // units per row
  const int units = F * nur;   // units per sample
  const int G = gridDim.x;
  const int last = B - 1;

  // per table (lane t < F): first joint-table row and row count
  uint32_t tbase = 0, trows = 1;
  if (lane < F) {
    tbase = static_cast<uint32_t>(row_off[lane]);
    trows = static_cast<uint32_t>(row_off[lane + 1] - row_off[lane]);
  }
  // CSR bounds of sample j's bag in table `lane`.  The bounds (and the first indices) of 32
  // neighbouring samples share a 128-byte line that 32 different wavefronts read, so these
  // are plain loads that leave the line in L2 for all of them (non-temporal loads here made
  // the kernel 1.3-1.6x slower: fwd_core 170 -> 134 us, large_table 538 -> 366 us as plain)
  auto clampj = [&](int j) { return j < 0 ? 0 : (j < last ? j : last); };
  auto load_bounds = [&](int j, int& s, int& e) {
    const int g = (lane < F ? lane : 0) * B + clampj(j);
    s = off[g];
    e = off[g + 1];
  };
  // first index of the bag (any valid position when the bag is empty)
  auto load_first = [&](int s) -> int32_t {
    return idx[s < 0 ? 0 : (s < nnz ? s : nnz - 1)];
  };
  // joint-table row of the first entry (row 0 for an empty bag: read, never used)
  auto first_row = [&](int32_t r, int s, int e) -> uint32_t {
    if (hash) r = floor_mod(r, static_cast<int32_t>(trows));
    return e > s ? tbase + static_cast<uint32_t>(r) : 0u;
  };
  auto issue_rows = [&](int j, uint32_t rid, Unit<TT> (&rows)[NU], u32x4& xv) {
    const int jc = clampj(j);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      int q = u * 64 + lane;
      q = q < units ? q : units - 1;
      const int t = q / nur, c = q - t * nur;
      const uint32_t r = static_cast<uint32_t>(__shfl(static_cast<int>(rid), t));
      load_unit<TT>(rows[u], W + static_cast<int64_t>(r) * D + c * 8);
    }
    const int xc = lane < nur ? lane : nur - 1;
    xv = *reinterpret_cast<const u32x4*>(x0 + static_cast<int64_t>(jc) * D + xc * 8);
  };

  // prologue: bounds of samples j, j+G, j+2G; first indices of j, j+G; rows of j.  All of
  // it lands before the loop starts (settle), so that the wait counts the compiler derives
  // for the loop are those of its steady state alone.
  // samples handed to the XCDs in contiguous runs, so that the wavefronts sharing a line of
  // bounds or indices share one L2 (fwd_core 134 -> 130 us, large_table 366 -> 349 us)
  int j = (G & 7) == 0 ? xcd_remap(blockIdx.x, G) : static_cast<int>(blockIdx.x);
  int s0, e0, s1, e1, s2, e2;
  load_bounds(j, s0, e0);
  load_bounds(j + G, s1, e1);
  load_bounds(j + 2 * G, s2, e2);
  int32_t r1 = load_first(s1);
  Unit<TT> rows[NU];
  u32x4 xv;
  issue_rows(j, first_row(load_first(s0), s0, e0), rows, xv);
#pragma unroll
  for (int u = 0; u < NU; ++u)
#pragma unroll
    for (int i = 0; i < Unit<TT>::NV; ++i) settle(rows[u].v[i]);
  settle(xv);
  settle(s1); settle(e1); settle(s2); settle(e2); settle(r1);

  for (; j < B; j += G) {
    // (1) bounds of sample j+3G, first indices of sample j+2G
    int s3, e3;
    load_bounds(j + 3 * G, s3, e3);
    const int32_t r2 = load_first(s2);

    // (2) pool sample j: first rows (in registers), further entries of multi-hot bags in CSR
    //     order, fp32; one rounding to the activation type, straight into the LDS tile
    //     (rows 1..); x0 into row 0
    const int nonempty = e0 > s0;
    if (__ballot(lane < F && e0 - s0 > 1) == 0) {  // wave-uniform: hotness <= 1
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        int q = u * 64 + lane;
        q = q < units ? q : units - 1;  // lanes past the end repeat the last unit (same bytes)
        const int t = q / nur, c = q - t * nur;
        const bool ne = __shfl(nonempty, t) != 0;
        float f[8];
        unit_to_f<TT>(rows[u], f);
#pragma unroll
        for (int x = 0; x < 8; ++x) f[x] = ne ? f[x] : 0.0f;
        *reinterpret_cast<u32x4*>(lds + (1 + t) * pitch + c * 16) = pack8<IT>(f);
      }
    } else {  // multi-hot bags: the further entries four at a time (all their loads in flight)
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        int q = u * 64 + lane;
        q = q < units ? q : units - 1;
        const int t = q / nur, c = q - t * nur;
        const bool ne = __shfl(nonempty, t) != 0;
        const int bs = __shfl(s0, t), be = __shfl(e0, t);
        const uint32_t tb = static_cast<uint32_t>(__shfl(static_cast<int>(tbase), t));
        const int32_t nt = __shfl(static_cast<int>(trows), t);
        float f[8];
        unit_to_f<TT>(rows[u], f);
        for (int k = bs + 1; k < be; k += 4) {
          // indices, then rows, of the next four entries (entries past the bag's end re-read
          // its last entry and are not added); added in CSR order
          int32_t r[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            r[e] = idx[k + e < be ? k + e : be - 1];
            if (hash) r[e] = floor_mod(r[e], nt);
          }
          Unit<TT> w[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            load_unit<TT>(w[e], W + static_cast<int64_t>(tb + static_cast<uint32_t>(r[e])) * D + c * 8);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (k + e < be) {
              float g[8];
              unit_to_f<TT>(w[e], g);
#pragma unroll
              for (int x = 0; x < 8; ++x) f[x] += g[x];
            }
          }
        }
#pragma unroll
        for (int x = 0; x < 8; ++x) f[x] = ne ? f[x] : 0.0f;
        *reinterpret_cast<u32x4*>(lds + (1 + t) * pitch + c * 16) = pack8<IT>(f);
      }
    }
    *reinterpret_cast<u32x4*>(lds + (lane < nur ? lane * 16 : trash)) = xv;

    // (3) rows of sample j+G (their first indices were loaded one trip ago) -- issued
    //     before this trip's stores
    issue_rows(j + G, first_row(r1, s1, e1), rows, xv);

    // (4) the interaction: x0 copy, zero padding, strict lower triangle of the Gram matrix
    __syncthreads();
    for (int d = lane; d < D; d += 64)
      ostage[d] = IT::from_f(IT::to_f(*reinterpret_cast<const uint16_t*>(lds + d * 2)));
    for (int c = D + P + lane; c < out_stride; c += 64) ostage[c] = 0;
    gram_lower_to_lds<IT, IT>(lds, pitch, V, D, obase, trash);
    __syncthreads();

    // (5) the output row: a fixed number of 16-byte stores per lane
    uint16_t* orow = out + static_cast<int64_t>(j) * out_stride;
    const int nchunk = obytes / 16;
#pragma unroll
    for (int k = 0; k < SPL; ++k) {
      int q = k * 64 + lane;
      q = q < nchunk ? q : nchunk - 1;
      reinterpret_cast<u32x4*>(orow)[q] = reinterpret_cast<const u32x4*>(ostage)[q];
    }

    s0 = s1; e0 = e1;
    s1 = s2; e1 = e2;
    s2 = s3; e2 = e3;
    r1 = r2;
  }
}

template <class TT, class IT, int NU, int SPL>
el_status launch_t(const el_tables& tab, const el_bags& bags, uint32_t flags, const void* x0,
                   void* out, int out_stride, size_t lds, hipStream_t stream) {
  auto kern = k_emb_dot_fwd<TT, IT, NU, SPL>;
  const int B = bags.batch;
  // twice the workgroups that fit at once when each still loops over 16 samples or more:
  // late or slow ones hand their samples to the dispatcher instead of holding up the end
  // (fwd_core 174 -> 170 us, large_table 551 -> 496 us at B = 262144; with fewer samples
  // per workgroup the extra ones cost more than they balance: B = 4096 16 -> 18 us, and four
  // times the grid lost at B = 1048576, 2.29 -> 2.57 ms)
  const int64_t resident = resident_grid(reinterpret_cast<const void*>(kern), B, lds, 64);
  const int64_t grid = B >= 32 * resident ? 2 * resident : resident;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)),
                     dim3(64), lds, stream, static_cast<const typename TT::S*>(tab.base),
                     tab.row_offset, bags.indices, static_cast<int32_t>(bags.nnz), bags.offsets, B,
                     tab.num_tables, tab.dim, (flags & EL_FLAG_HASH_INDICES) ? 1u : 0u,
                     static_cast<const uint16_t*>(x0), static_cast<uint16_t*>(out), out_stride);
  return check_launch("emb_dot_fwd");
}

// Shape classes: row units per lane (NU) and output-row chunks per lane (SPL).
template <class TT, class IT>
el_status launch_shape(const el_tables& tab, const el_bags& bags, uint32_t flags, const void* x0,
                       void* out, int out_stride, size_t lds, hipStream_t stream) {
  const int units = tab.num_tables * (tab.dim / 8);
  const int ochunks = (out_stride * 2 + 15) / 16;
#define EL_SPL(NU)                                                                                   \
  do {                                                                                               \
    if (ochunks <= 64) return launch_t<TT, IT, NU, 1>(tab, bags, flags, x0, out, out_stride, lds, stream); \
    if (ochunks <= 256) return launch_t<TT, IT, NU, 4>(tab, bags, flags, x0, out, out_stride, lds, stream); \
  } while (0)
  if (units <= 2 * 64) EL_SPL(2);
  else if (units <= 4 * 64) EL_SPL(4);
  else if (units <= 7 * 64) EL_SPL(7);
  else if (units <= 12 * 64) EL_SPL(12);
  else if (units <= 16 * 64) EL_SPL(16);
#undef EL_SPL
  return set_error(EL_ERR_UNSUPPORTED,
                   "emb_dot_fwd: without emb_out the fused kernel covers F * D / 8 <= 1024 row chunks "
                   "and output rows of at most 4096 bytes");
}

template <class TT>
el_status launch_act(const el_tables& tab, const el_bags& bags, uint32_t flags, const void* x0,
                     el_dtype act, void* out, int out_stride, size_t lds,
                     hipStream_t stream) {
  if (act == EL_BF16) return launch_shape<TT, BF16T>(tab, bags, flags, x0, out, out_stride, lds, stream);
  if (act == EL_F16) return launch_shape<TT, F16T>(tab, bags, flags, x0, out, out_stride, lds, stream);
  return set_error(EL_ERR_UNSUPPORTED, "emb_dot_fwd: without emb_out the activations must be bf16 or fp16");
}

}  // namespace

// With emb_out: the gather (table-major, for its L2 locality) and the interaction run on
// chunks of samples whose pooled vectors fit in the memory-side cache, each chunk's
// interaction right after its gather, so that the pooled vectors are read back from that
// cache rather than from HBM.  Without emb_out: the fused kernel, which covers 16-bit
// activations, D % 16 == 0, F <= 64, 16-byte output rows and a tile that fits in LDS
// (EL_ERR_UNSUPPORTED, nothing enqueued, otherwise).
el_status launch_emb_dot_fwd(const el_tables& tab, const el_bags& bags, uint32_t flags,
                             const void* x0, el_dtype act_dtype, void* emb_out, void* out,
                             int out_stride, hipStream_t stream) {
  const int F = tab.num_tables, D = tab.dim, B = bags.batch;
  if (emb_out) {
    constexpr int64_t kChunkBytes = 224ll << 20;  // below the 256 MB memory-side cache
    const int64_t es = static_cast<int64_t>(dtype_size(act_dtype));
    const int64_t per = static_cast<int64_t>(F) * D * es;  // pooled bytes per sample
    const int64_t nch = (per * B + kChunkBytes - 1) / kChunkBytes;
    const int chunk = static_cast<int>((B + nch - 1) / nch);
    for (int b0 = 0; b0 < B; b0 += chunk) {
      const int bc = B - b0 < chunk ? B - b0 : chunk;
      el_status st = launch_emb_bag_fwd(tab, bags, flags, emb_out, act_dtype, stream, b0, bc);
      if (st != EL_OK) return st;
      const int64_t b = b0;
      st = launch_dot_fwd(static_cast<const char*>(x0) + b * D * es,
                          static_cast<const char*>(emb_out) + b * per, act_dtype, bc, F, D,
                          static_cast<char*>(out) + b * out_stride * es,
                          act_dtype, out_stride, stream);
      if (st != EL_OK) return st;
    }
    return EL_OK;
  }
  const size_t V = static_cast<size_t>(F) + 1;
  const size_t obytes = (static_cast<size_t>(out_stride) * 2 + 15) / 16 * 16;
  const size_t lds = V * (D * 2 + 16) + obytes + 16;
  if (act_dtype == EL_F32 || D % 16 != 0 || F > 64 || (out_stride * 2) % 16 != 0 ||
      lds > 64 * 1024 || bags.nnz == 0 || tab.total_rows == 0)
    return set_error(EL_ERR_UNSUPPORTED, "emb_dot_fwd: without emb_out the shape must suit the fused "
                                         "kernel (16-bit activations, D % 16 == 0, F <= 64, 16-byte rows)");
  switch (tab.dtype) {
    case EL_F32: return launch_act<F32T>(tab, bags, flags, x0, act_dtype, out, out_stride, lds, stream);
    case EL_F16: return launch_act<F16T>(tab, bags, flags, x0, act_dtype, out, out_stride, lds, stream);
    case EL_BF16: return launch_act<BF16T>(tab, bags, flags, x0, act_dtype, out, out_stride, lds, stream);
    default: break;
  }
  return set_error(EL_ERR_INVALID_ARG, "emb_dot_fwd: unknown table dtype");
}

}  // namespace el
