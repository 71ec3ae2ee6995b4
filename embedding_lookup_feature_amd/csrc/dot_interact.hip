// dot_interact.hip -- pairwise "dot interaction" forward and backward (gfx950).
//
// Page "DLRM For PyTorch", §Model architecture: the bottom-MLP output and the embedding
// vectors of a sample are fed to a dot interaction, whose output is concatenated with the
// bottom-MLP output.  With V = F+1 vectors per sample (vector 0 = x0[b], vector 1+t = the
// pooled embedding of table t) the interaction is the strict lower triangle of the Gram
// matrix Z = V V^T, stored row-major: pair (i, j), i > j, at p(i,j) = i(i-1)/2 + j.
//
// 16-bit inputs (bf16 / fp16): one wavefront per sample.  The sample's V x D tile is
// streamed from HBM with 16-byte loads into LDS (non-temporal in the forward, whose
// wavefronts each cover whole rows; the backward's lanes each take one chunk of many rows,
// so a cache line feeds several of its load instructions and stays with the default
// policy; row pitch padded by 16 bytes so that the
// 32 rows read by one MFMA operand fall on distinct banks), then
//   forward : the lower-triangular 32x32 tiles of Z are v_mfma_f32_32x32x16_{bf16,f16}
//             products of the tile with itself, K = D in steps of 16 (fp32 accumulate);
//   backward: dV = S V with the symmetric pair-gradient matrix S, as MFMA products of S
//             (rebuilt from the staged gradient row) and V (read transposed from LDS).
// The contraction index of each MFMA is assigned the same way in both operands, so the
// result does not depend on how the hardware orders K inside one instruction.
// fp32 inputs (and shapes the MFMA path does not cover) use an fp32 FMA kernel.
#include <algorithm>
#include <map>
#include <mutex>
#include <tuple>
#include <type_traits>
#include <utility>

#include "el_internal.hpp"
#include "el_mfma.hpp"

namespace el {

// Workgroups that loop over samples: launch as many as can be resident at once (occupancy
// from the kernel's registers and LDS), never more than there are samples.
int resident_grid(const void* kernel, int B, size_t lds_bytes, int block) {
  static std::mutex mu;
  static std::map<std::tuple<int, const void*, size_t>, int> cache;  // (device, kernel, LDS)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  int per_cu = 0;
  {
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find({dev, kernel, lds_bytes});
    if (it != cache.end()) {
      per_cu = it->second;
    } else {
      int n = 0, cus = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, block, lds_bytes) != hipSuccess) n = 4;
      if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 256;
      per_cu = (n > 0 ? n : 1) * (cus > 0 ? cus : 256);
      cache[{dev, kernel, lds_bytes}] = per_cu;
    }
  }
  return B < per_cu ? B : per_cu;
}

namespace {

__device__ inline int64_t pair_pos(int i, int j) { return static_cast<int64_t>(i) * (i - 1) / 2 + j; }

// One sample's inputs as a sequence of 16-byte chunks, lane-strided over the wavefront:
// chunks [0, tile) are the V x D tile (row 0 = x0[b], rows 1.. = emb[b], contiguous in
// memory), chunks [tile, total) the first elements of the upstream-gradient row
// (backward only).  All of a sample's loads are issued back to back into registers; the
// caller issues the next sample's loads before computing on the current one, so one
// sample's HBM latency hides behind the previous sample's MFMA work.  Lanes past the end
// re-load the last chunk (in bounds, no branch) and later write it to a scratch LDS slot.
template <int NQ, bool WITH_GRAD>
__device__ inline void fetch_sample(const uint16_t* __restrict__ x0, const uint16_t* __restrict__ emb,
                                    const uint16_t* __restrict__ dout, int out_stride, int b, int F,
                                    int D, int tile, int total, u32x4 (&r)[NQ]) {
  const int nv = D / 8;
  const int64_t x0_base = static_cast<int64_t>(b) * D;
  const int64_t emb_base = static_cast<int64_t>(b) * F * D - static_cast<int64_t>(nv) * 8;
  const int64_t g_base = static_cast<int64_t>(b) * out_stride - static_cast<int64_t>(tile) * 8;
#pragma unroll
  for (int u = 0; u < NQ; ++u) {
    int q = u * 64 + static_cast<int>(threadIdx.x & 63);
    q = q < total ? q : total - 1;
    const uint16_t* src;
    if constexpr (WITH_GRAD) {
      src = q < nv ? x0 + x0_base + q * 8 : (q < tile ? emb + emb_base + q * 8 : dout + g_base + q * 8);
    } else {
      src = q < nv ? x0 + x0_base + q * 8 : emb + emb_base + q * 8;
    }
    r[u] = ld_stream16(src);
  }
}

// Write the fetched chunks to LDS: tile rows at `pitch`-byte pitch from offset 0, gradient
// chunks packed from byte `goff`, chunks past the end to the scratch slot at `trash`.
template <int NQ>
__device__ inline void put_sample(char* lds, int pitch, int goff, int trash, int D, int tile,
                                  int total, const u32x4 (&r)[NQ]) {
  const int nv = D / 8;
#pragma unroll
  for (int u = 0; u < NQ; ++u) {
    const int q = u * 64 + static_cast<int>(threadIdx.x & 63);
    const int row = q / nv, c = q - row * nv;
    const int off = q < tile ? row * pitch + c * 16 : (q < total ? goff + (q - tile) * 16 : trash);
    *reinterpret_cast<u32x4*>(lds + off) = r[u];
  }
}


// ---------------------------------------------------------------------------------------
// Forward, MFMA path.  WPB independent wavefronts per workgroup, each with its own LDS
// region and its own samples (workgroups of several wavefronts let more wavefronts be
// resident per CU than one-wavefront workgroups do).
// LDS per wavefront: V x D tile (pitch 2D+16) | one output row (16-byte rounded) | 16-byte
// scratch slot.
// ---------------------------------------------------------------------------------------
// Orders this wavefront's LDS accesses around it (the wavefront's LDS operations execute in
// order; this keeps the compiler from moving them across).
__device__ inline void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <class IT, class OT, int NQ, int SPL, int WPB>
__global__ __launch_bounds__(64 * WPB) void k_dot_fwd_mfma(const uint16_t* __restrict__ x0,
                                                           const uint16_t* __restrict__ emb, int B,
                                                           int F, int D,
                                                           typename OT::S* __restrict__ out,
                                                           int out_stride, int vec_out,
                                                           int wave_lds) {
  extern __shared__ uint4 smem[];
  const int wave = threadIdx.x >> 6;
  char* lds = reinterpret_cast<char*>(smem) + wave * wave_lds;
  using OS = typename OT::S;
  const int V = F + 1;
  const int P = V * (V - 1) / 2;
  const int pitch = D * 2 + 16;
  const int obase = V * pitch;
  const int obytes = (out_stride * static_cast<int>(sizeof(OS)) + 15) / 16 * 16;
  const int trash = obase + obytes;
  OS* ostage = reinterpret_cast<OS*>(lds + obase);
  const int lane = threadIdx.x & 63;
  const int tile = V * (D / 8);
  const int stride = gridDim.x * WPB;

  u32x4 r[NQ];
  int b = blockIdx.x * WPB + wave;
  if (b < B) fetch_sample<NQ, false>(x0, emb, x0, 0, b, F, D, tile, tile, r);
  for (; b < B; b += stride) {
    put_sample<NQ>(lds, pitch, 0, trash, D, tile, tile, r);
    if (b + stride < B)
      fetch_sample<NQ, false>(x0, emb, x0, 0, b + stride, F, D, tile, tile, r);
    wave_sync();
    // x0 copy (converted to the output type; exact when the types agree) and zero padding
    for (int d = lane; d < D; d += 64)
      ostage[d] = OT::from_f(IT::to_f(*reinterpret_cast<const uint16_t*>(lds + d * 2)));
    for (int c = D + P + lane; c < out_stride; c += 64) ostage[c] = OT::from_f(0.0f);
    gram_lower_to_lds<IT, OT>(lds, pitch, V, D, obase, trash);
    wave_sync();
    OS* orow = out + static_cast<int64_t>(b) * out_stride;
    if (SPL > 0 && vec_out) {
      // a fixed number of 16-byte stores per lane (lanes past the end repeat the last chunk
      // with the same bytes), so that waiting for the next sample's loads never has to wait
      // for these stores as well
      const int nchunk = obytes / 16;
#pragma unroll
      for (int k = 0; k < SPL; ++k) {
        int q = k * 64 + lane;
        q = q < nchunk ? q : nchunk - 1;
        reinterpret_cast<u32x4*>(orow)[q] = reinterpret_cast<const u32x4*>(ostage)[q];
      }
    } else {
      for (int c = lane; c < out_stride; c += 64) orow[c] = ostage[c];
    }
  }
}

// ---------------------------------------------------------------------------------------
// Forward, MFMA path for many vectors (more than one 32-row tile per sample): the four
// wavefronts of a workgroup share one sample's V x D tile in LDS (pitch 2D+16), and the
// lower-triangular 32x32 tiles of Z are dealt out to them round-robin.  Each wavefront
// writes its products straight from the MFMA accumulators to the output row: for one
// accumulator register, lanes 0-31 hold 32 consecutive columns j of one row i and lanes
// 32-63 those of row i+4, so a store covers two runs of consecutive pair positions
// D + i(i-1)/2 + j.  No output row is staged in LDS, which leaves room for more resident
// samples than the one-wavefront-per-sample kernel.  The next sample's tile is loaded into
// registers before the current one is multiplied.
// ---------------------------------------------------------------------------------------
template <class IT, class OT, int NQ>
__global__ __launch_bounds__(256) void k_dot_fwd_wide(const uint16_t* __restrict__ x0,
                                                      const uint16_t* __restrict__ emb, int B,
                                                      int F, int D, typename OT::S* __restrict__ out,
                                                      int out_stride) {
  extern __shared__ uint4 smem[];
  char* lds = reinterpret_cast<char*>(smem);
  using OS = typename OT::S;
  const int V = F + 1;
  const int P = V * (V - 1) / 2;
  const int pitch = D * 2 + 16;
  const int trash = V * pitch;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, col = lane & 31;
  const int nv = D / 8;
  const int tile = V * nv;  // 16-byte chunks of a sample's vectors
  const int NT = (V + 31) / 32;
  const int ntiles = NT * (NT + 1) / 2;

  // chunk q of sample bb (q < tile: row q / nv of the V x D tile, contiguous from x0[bb]
  // and emb[bb]); chunks past the tile re-load the last one
  u32x4 r[NQ];
  auto fetch = [&](int bb) {
    const int64_t x0b = static_cast<int64_t>(bb) * D;
    const int64_t eb = static_cast<int64_t>(bb) * F * D - D;
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      int q = u * 256 + tid;
      q = q < tile ? q : tile - 1;
      const int row = q / nv, c = q - row * nv;
      const uint16_t* src = row == 0 ? x0 + x0b + c * 8 : emb + eb + static_cast<int64_t>(row) * D + c * 8;
      r[u] = ld_stream16(src);
    }
  };
  int b = blockIdx.x;
  if (b >= B) return;
  fetch(b);
  for (; b < B; b += gridDim.x) {
    __syncthreads();  // the previous sample's products have read the tile
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      const int q = u * 256 + tid;
      const int row = q / nv, c = q - row * nv;
      *reinterpret_cast<u32x4*>(lds + (q < tile ? row * pitch + c * 16 : trash)) = r[u];
    }
    if (b + static_cast<int>(gridDim.x) < B) fetch(b + gridDim.x);
    __syncthreads();
    OS* orow = out + static_cast<int64_t>(b) * out_stride;
    // x0 copy (converted to the output type; exact when the types agree) and zero padding
    for (int d = tid; d < D; d += 256) orow[d] = OT::from_f(IT::to_f(*reinterpret_cast<const uint16_t*>(lds + d * 2)));
    for (int c = D + P + tid; c < out_stride; c += 256) orow[c] = OT::from_f(0.0f);
    for (int t = wave; t < ntiles; t += 4) {  // wave-uniform
      int I = 0, J = t;
      while (J > I) { J -= I + 1; ++I; }
      f32x16 acc = {};
      const int ra = I * 32 + col, rb = J * 32 + col;
      for (int ks = 0; ks < D / 16; ++ks) {
        const int cb = (2 * ks + half) * 16;  // byte offset of this lane's 8 elements
        const u32x4 a = lds16_or_zero(lds, ra * pitch + cb, ra < V);
        const u32x4 bv = (I == J) ? a : lds16_or_zero(lds, rb * pitch + cb, rb < V);
        acc = mfma32<IT>(a, bv, acc);
      }
      const int j = J * 32 + col;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int i = I * 32 + acc_row(rr, lane);
        if (i < V && j < i) orow[D + i * (i - 1) / 2 + j] = OT::from_f(acc[rr]);
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// Backward, MFMA path, computed transposed: dV^T = V^T S (S is symmetric), so that
//   A = V^T  (lane: one dimension d, 8 consecutive vectors)  -> one 16-byte LDS read,
//   B = S    (lane: one vector v, 8 consecutive vectors)     -> rebuilt from the gradient row,
//   C = dV^T (lane: one vector v, runs of 4 consecutive d)   -> 8-byte LDS writes.
// A workgroup of 4 wavefronts works on one sample at a time (grid-strided over samples,
// the loads of the sample PD strides ahead issued before the current one is computed,
// into one of PD register buffers).  Loading: every
// thread takes pairs of rows of one 8-element column block (2 x 16-byte loads), interleaves
// them into 8 two-vector words and writes those into V^T.  Compute: the 32 x 32 output
// tiles (vector tile, dimension tile) are dealt round-robin to the 4 wavefronts.  Store:
// all threads write the V x D block with 16-byte stores; dx0 = G[0:D) + dV_0 is formed
// there from an fp32 copy of dV_0 and the G[0:D) chunk each thread read into registers
// before the barrier that ends the compute (the gradient row's LDS bytes are rewritten by
// the next sample's fill once a wavefront passes that barrier, so nothing reads them after
// it).  dout has the input's 16-bit type (S is then exact).
// LDS: V^T [D][VP] | gradient row | VP x D output block | dV_0 in fp32 | scratch slot.
// UPT: row pairs per thread; GPT: gradient-row chunks per thread held in registers
// (0: loaded straight into LDS when the sample starts); KSM: K steps (>= KS); PD: samples
// in flight per workgroup (1, or 2 with GPT > 0: a third measured no faster).
// Workgroups per CU the register budget is set for: four for one row pair per thread
// (117 VGPRs, measured faster than three), two for the gather variant and for three
// register-held gradient chunks (at most 256 VGPRs), otherwise what the kernel needs.
// ---------------------------------------------------------------------------------------
template <int N>
using Buf = std::integral_constant<int, N>;

// An empty register use: the compiler waits here for the load that produced `v`.
__device__ inline void settle(const u32x4& v) { asm volatile("" ::"v"(v)); }
__device__ inline void settle_i(int v) { asm volatile("" ::"v"(v)); }

// GATHER: the pooled vectors are rebuilt from the tables (TT: table type) instead of read
// from emb, exactly as emb_bag_fwd forms them: the bag's rows summed in fp32 in CSR order
// (starting from the first row; an empty bag is +0), one rounding to IT.  Each thread
// resolves its own two rows through a three-stage pipeline over the grid stride: the table
// rows of the sample 2 strides ahead, its first index 4 strides ahead, its CSR bounds 6
// strides ahead, each stage consuming what the previous stage loaded two trips earlier (the
// register sets alternate with the trips), so every load has two trips to arrive.  The
// further rows of a bag longer than one are loaded where the tile is written
// to LDS (synchronously: correct for any bag, fast for one-lookup bags).
struct GatherSrc {
  const void* W;            // joint table [total_rows][D] of TT
  const int64_t* row_off;   // [F+1]
  const int32_t* idx;       // [nnz]
  const int32_t* off;       // [F*B+1]
  int32_t nnz;
  uint32_t hash;            // floor-mod the indices by the table's row count
};

template <int UPT, int GPT, bool GATHER>
constexpr int bwd_wg_per_cu() { return GATHER ? 2 : (UPT == 1 ? 4 : (GPT == 3 ? 2 : 1)); }

template <class IT, class GT, int UPT, int GPT, int KSM, int PD, class TT, bool GATHER>
__global__ __launch_bounds__(256, (bwd_wg_per_cu<UPT, GPT, GATHER>())) void k_dot_bwd_mfma(
    const uint16_t* __restrict__ x0, const uint16_t* __restrict__ emb, int B, int F, int D,
    const uint16_t* __restrict__ dout, int out_stride, typename GT::S* __restrict__ dx0,
    typename GT::S* __restrict__ demb, GatherSrc gs) {
  extern __shared__ uint4 smem[];
  char* lds = reinterpret_cast<char*>(smem);
  using GS = typename GT::S;
  constexpr int GSZ = static_cast<int>(sizeof(GS));
  const int V = F + 1;
  const int P = V * (V - 1) / 2;
  const int NT = (V + 31) / 32;
  const int VP = NT * 32;
  const int DT = (D + 31) / 32;  // D % 16 == 0; a last tile of 16 rows is half empty
  const int tpitch = VP * 2 + 16;
  // DS (gradient row in registers, up to 128 vectors): S is built densely in LDS from the
  // registers and only the gradient row's first D elements (dx0's direct term) are kept;
  // otherwise the whole gradient row is staged and S is read from it element by element
  constexpr bool DS = GPT == 3;
  const int goff = D * tpitch;
  const int gchunks = (D + P + 7) / 8;
  const uint16_t* G = reinterpret_cast<const uint16_t*>(lds + goff);
  const int spitch = VP * 2 + 16;  // dense S row pitch (DS)
  const int soff = goff + D * 2;   // D % 16 == 0: 16-byte aligned
  const int opitch = D * GSZ + 16;
  const int ooff = DS ? soff + VP * spitch : goff + gchunks * 16;
  const int r0off = ooff + VP * opitch;  // dV_0, fp32
  const int trash = r0off + D * 4;
  const int KS = (V + 15) / 16;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, col = lane & 31;
  const int npairs = VP / 2;
  const int units = npairs * (D / 8);  // (row pair, column block); row pair fastest

  static_assert(PD == 1 || (PD == 2 && GPT > 0),
                "several samples in flight need the gradient row in registers");
  static_assert(!GATHER || PD == 2, "the gather pipeline is built for two samples in flight");
  using TS = typename TT::S;
  // 16-byte vectors per 8-element row chunk: a table chunk of TT when gathering
  constexpr int NVT = GATHER ? static_cast<int>(sizeof(TS)) / 2 : 1;
  u32x4 t[PD][UPT][2][NVT];
  u32x4 g[PD][GPT > 0 ? GPT : 1];

  // Gather state of this thread's rows (uu, m): table row base and count, and per pipeline
  // parity: CSR bounds, first index with its bag's length, and the length of the bag whose
  // first rows sit in register buffer `parity`.
  constexpr int GU = GATHER ? UPT : 1;
  uint32_t tb[GU][2] = {}, tr[GU][2] = {};
  int bnd_s[2][GU][2] = {}, bnd_e[2][GU][2] = {}, gix[2][GU][2] = {};
  int ibag_n[2][GU][2] = {}, bag_n[2][GU][2] = {};
  // table of row (uu, m), or -1 for x0 / padding rows
  auto row_table = [&](int uu, int m) {
    int u = uu * 256 + tid;
    u = u < units ? u : units - 1;
    const int rp = u - (u / npairs) * npairs;
    const int v = rp * 2 + m;
    return v >= 1 && v < V ? v - 1 : -1;
  };
  const int lastb = B - 1;
  // stage A: CSR bounds of sample j's bags (padding rows read bag 0's)
  auto g_bounds = [&](int j, auto par) {
    constexpr int Q = decltype(par)::value;
    const int jc = j < lastb ? j : lastb;
#pragma unroll
    for (int uu = 0; uu < GU; ++uu)
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int tt = row_table(uu, m);
        const int gbag = (tt < 0 ? 0 : tt) * B + jc;
        // plain loads: 32 neighbouring samples' bounds (and first indices) share a cache
        // line that as many wavefronts read (streamed, the call took 553 instead of 409 us)
        bnd_s[Q][uu][m] = gs.off[gbag];
        bnd_e[Q][uu][m] = gs.off[gbag + 1];
      }
  };
  // stage B: first index of the bags whose bounds are in parity Q's registers (the bag's
  // length moves along with it)
  auto g_first = [&](auto par) {
    constexpr int Q = decltype(par)::value;
#pragma unroll
    for (int uu = 0; uu < GU; ++uu)
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        int p = bnd_s[Q][uu][m];
        ibag_n[Q][uu][m] = bnd_e[Q][uu][m] - p;
        p = p < 0 ? 0 : (p < gs.nnz ? p : gs.nnz - 1);
        gix[Q][uu][m] = gs.idx[p];
      }
  };
  // joint-table row of a bag's first index (row 0 for an empty bag: read, never used)
  auto g_row = [&](int uu, int m, int r, int n) -> uint32_t {
    if (gs.hash) r = floor_mod(r, static_cast<int32_t>(tr[uu][m]));
    return n > 0 ? tb[uu][m] + static_cast<uint32_t>(r) : 0u;
  };

  // Loads of sample bb into register buffer BF (GATHER: the first rows of the bags whose
  // indices are in parity BF's registers, which are sample bb's).
  auto fetch = [&](int bb, auto bf) {
    constexpr int BF = decltype(bf)::value;
    const int64_t xb = static_cast<int64_t>(bb) * D;
    const int64_t eb = static_cast<int64_t>(bb) * F * D - D;  // row v >= 1 at eb + v * D
#pragma unroll
    for (int uu = 0; uu < UPT; ++uu) {
      int u = uu * 256 + tid;
      u = u < units ? u : units - 1;
      const int c = u / npairs, rp = u - c * npairs;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int v = rp * 2 + m;
        const int vc = v < V ? v : 0;
        if constexpr (GATHER) {
          // vector 0: x0's chunk for row 0 (and padding rows), else the table chunk
          const bool trow = vc != 0;
          bag_n[BF][uu][m] = ibag_n[BF][uu][m];
          const uint32_t rid = g_row(uu, m, gix[BF][uu][m], bag_n[BF][uu][m]);
          const char* tsrc = reinterpret_cast<const char*>(static_cast<const TS*>(gs.W) +
                                                           static_cast<int64_t>(rid) * D + c * 8);
          const char* xsrc = reinterpret_cast<const char*>(x0 + xb + c * 8);
#pragma unroll
          for (int q = 0; q < NVT; ++q)
            t[BF][uu][m][q] = *reinterpret_cast<const u32x4*>(trow ? tsrc + 16 * q : xsrc);
        } else {
          const uint16_t* src = (vc == 0 ? x0 + xb : emb + eb + static_cast<int64_t>(vc) * D) + c * 8;
          t[BF][uu][m][0] = *reinterpret_cast<const u32x4*>(src);  // rows >= V are masked in put()
        }
      }
    }
    if constexpr (GPT > 0) {
      const int64_t gb = static_cast<int64_t>(bb) * out_stride;
#pragma unroll
      for (int gg = 0; gg < GPT; ++gg) {
        int q = gg * 256 + tid;
        q = q < gchunks ? q : gchunks - 1;
        g[BF][gg] = *reinterpret_cast<const u32x4*>(dout + gb + q * 8);
      }
    }
  };
  auto settle_buf = [&](auto bf) {
    constexpr int BF = decltype(bf)::value;
#pragma unroll
    for (int uu = 0; uu < UPT; ++uu)
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int q = 0; q < NVT; ++q) settle(t[BF][uu][m][q]);
    if constexpr (GPT > 0) {
#pragma unroll
      for (int gg = 0; gg < GPT; ++gg) settle(g[BF][gg]);
    }
  };
  // GATHER: the pooled 8-element chunk of row (uu, m) as IT: the bag's first row (loaded
  // into buffer BF by the pipeline), plus its further rows in CSR order (loaded here), in
  // fp32 -- the association emb_bag_fwd uses; an empty bag pools to +0.
  auto pooled = [&](int uu, int m, int c, int bb, auto bf) -> u32x4 {
    constexpr int BF = decltype(bf)::value;
    float acc[8];
    const int n = bag_n[BF][uu][m];
#pragma unroll
    for (int q = 0; q < NVT; ++q) {
      const u32x4 w = n > 0 ? t[BF][uu][m][q] : u32x4{0, 0, 0, 0};
      unpack16<TT>(uint4{w[0], w[1], w[2], w[3]}, acc + q * epv<TT>());
    }
    if (n > 1) {
      const int s0 = gs.off[row_table(uu, m) * B + min(bb, B - 1)];
      for (int k = s0 + 1; k < s0 + n; ++k) {
        const uint32_t rid = g_row(uu, m, gs.idx[k], 1);
        const TS* src = static_cast<const TS*>(gs.W) + static_cast<int64_t>(rid) * D + c * 8;
#pragma unroll
        for (int q = 0; q < NVT; ++q) {
          const uint4 w = reinterpret_cast<const uint4*>(src)[q];
          float f[8];
          unpack16<TT>(w, f);
#pragma unroll
          for (int x = 0; x < epv<TT>(); ++x) acc[q * epv<TT>() + x] += f[x];
        }
      }
    }
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      r[i] = static_cast<uint32_t>(IT::from_f(acc[2 * i])) | (static_cast<uint32_t>(IT::from_f(acc[2 * i + 1])) << 16);
    return r;
  };

  // Register buffer BF (sample bb) -> LDS.
  auto put = [&](int bb, auto bf) {
    constexpr int BF = decltype(bf)::value;
#pragma unroll
    for (int uu = 0; uu < UPT; ++uu) {
      const int u = uu * 256 + tid;
      const int c = u / npairs, rp = u - c * npairs;
      u32x4 r0 = rp * 2 < V ? t[BF][uu][0][0] : u32x4{0, 0, 0, 0};
      u32x4 r1 = rp * 2 + 1 < V ? t[BF][uu][1][0] : u32x4{0, 0, 0, 0};
      if constexpr (GATHER) {
        if (u < units) {
          if (rp * 2 >= 1 && rp * 2 < V) r0 = pooled(uu, 0, c, bb, bf);
          if (rp * 2 + 1 < V) r1 = pooled(uu, 1, c, bb, bf);
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // value e of both rows, row 2rp in the low half: V^T[c*8 + e][2rp .. 2rp+1]
        const uint32_t a = r0[e >> 1], w = r1[e >> 1];
        const uint32_t word = (e & 1) ? __builtin_amdgcn_perm(w, a, 0x07060302u)
                                      : __builtin_amdgcn_perm(w, a, 0x05040100u);
        const int off = u < units ? (c * 8 + e) * tpitch + rp * 4 : trash;
        *reinterpret_cast<uint32_t*>(lds + off) = word;
      }
    }
    if constexpr (DS) {
      // chunk q holds elements 8q .. 8q+7 of the gradient row: the direct term (q < D/8,
      // kept for dx0) or pairs p = element - D, each written to S[i][j] and S[j][i]
      // (p = i(i-1)/2 + j, j < i); the diagonal and the padding of S stay zero
#pragma unroll
      for (int gg = 0; gg < GPT; ++gg) {
        const int q = gg * 256 + tid;
        if (q < D / 8) {
          *reinterpret_cast<u32x4*>(lds + goff + q * 16) = g[BF][gg];
        } else if (q < gchunks) {
          int p = q * 8 - D;
          int i = static_cast<int>((1.0f + sqrtf(1.0f + 8.0f * static_cast<float>(p))) * 0.5f);
          while (i * (i - 1) / 2 > p) --i;
          while ((i + 1) * i / 2 <= p) ++i;
          int j = p - i * (i - 1) / 2;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            if (p + e < P) {
              const uint16_t sv = static_cast<uint16_t>(g[BF][gg][e >> 1] >> ((e & 1) * 16));
              *reinterpret_cast<uint16_t*>(lds + soff + i * spitch + j * 2) = sv;
              *reinterpret_cast<uint16_t*>(lds + soff + j * spitch + i * 2) = sv;
            }
            if (++j == i) {
              ++i;
              j = 0;
            }
          }
        }
      }
    } else if constexpr (GPT > 0) {
#pragma unroll
      for (int gg = 0; gg < GPT; ++gg) {
        const int q = gg * 256 + tid;
        *reinterpret_cast<u32x4*>(lds + (q < gchunks ? goff + q * 16 : trash)) = g[BF][gg];
      }
    } else {
      // four chunks per thread in flight at once (clamped loads, masked LDS writes)
      const uint16_t* grow = dout + static_cast<int64_t>(bb) * out_stride;
      for (int q0 = 0; q0 < gchunks; q0 += 4 * 256) {
        u32x4 gv[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int q = q0 + k * 256 + tid;
          gv[k] = *reinterpret_cast<const u32x4*>(grow + (q < gchunks ? q : gchunks - 1) * 8);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int q = q0 + k * 256 + tid;
          *reinterpret_cast<u32x4*>(lds + (q < gchunks ? goff + q * 16 : trash)) = gv[k];
        }
      }
    }
  };

  // One sample: LDS fill from buffer BF, that buffer refilled with the sample PD strides
  // on (clamped to the last sample, so that every trip issues the same loads and stores
  // and the compiler's wait counts stay exact), compute, store.
  const int NG = gridDim.x;
  auto sample = [&](int b, auto bf) {
    put(b, bf);
    // GATHER: every stage consumes what the same stage of the trip before last (same
    // parity) loaded, so each load has two trips to arrive
    fetch(min(b + PD * NG, B - 1), bf);               // rows (GATHER: stage C), sample b + 2 NG
    if constexpr (GATHER) {
      g_first(bf);                                    // stage B: sample b + 4 NG
      g_bounds(b + 6 * NG, bf);                       // stage A: sample b + 6 NG
    }
    __syncthreads();
    int cur_vt = -1;
    u32x4 Sop[KSM];  // S[v][k], k = 16 ks + 8 half + e
    // each wavefront takes a run of consecutive tiles in row-tile-major order, so that it
    // builds the S operand of a row tile once and reuses it across the column tiles
    const int tpw = (NT * DT + 3) / 4;
    const int tile_end = min((wave + 1) * tpw, NT * DT);
    for (int tile = wave * tpw; tile < tile_end; ++tile) {
      const int vt = tile / DT, dt = tile - vt * DT;
      const int v = vt * 32 + col;
      if (vt != cur_vt && DS) {  // wave-uniform: S[v][16 ks + 8 half ..], one aligned read
        cur_vt = vt;
#pragma unroll
        for (int ks = 0; ks < KSM; ++ks)
          Sop[ks] = *reinterpret_cast<const u32x4*>(lds + soff + v * spitch + (ks * 16 + half * 8) * 2);
      } else if (vt != cur_vt) {  // wave-uniform
        cur_vt = vt;
#pragma unroll
        for (int ks = 0; ks < KSM; ++ks) {
          uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int k = ks * 16 + half * 8 + e;
            const bool ok = v < V && k < V && v != k;
            const int hi = v > k ? v : k, lo = v > k ? k : v;
            const uint32_t sv = G[ok ? D + hi * (hi - 1) / 2 + lo : 0];
            w[e >> 1] |= (ok ? sv : 0u) << ((e & 1) * 16);
          }
          Sop[ks] = u32x4{w[0], w[1], w[2], w[3]};
        }
      }
      f32x16 acc = {};
      const int arow = (dt * 32 + col) * tpitch + half * 16;
      const bool dok = dt * 32 + col < D;  // rows of V^T past D are zero
#pragma unroll
      for (int ks = 0; ks < KSM; ++ks)
        if (ks < KS) acc = mfma32<IT>(lds16_or_zero(lds, arow + ks * 32, dok), Sop[ks], acc);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int d0 = dt * 32 + q * 8 + half * 4;
        if (d0 < D) {
          float f[4] = {acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
          store_n<GT, 4>(reinterpret_cast<GS*>(lds + ooff + v * opitch + d0 * GSZ), f);
          if (v == 0) store_n<F32T, 4>(reinterpret_cast<float*>(lds + r0off + d0 * 4), f);
        }
      }
    }
    // dx0's direct term G[0:D): every thread takes gradient-row chunk qd into registers
    // before the barrier below.  After that barrier no thread reads the gradient row: a
    // wavefront that runs ahead may already be writing the next sample's row into the same
    // LDS bytes (put()), and the barrier is the last one it waits at before doing so.
    const int nd = D / 8;
    const int qd = tid < nd ? tid : nd - 1;  // threads past D/8 repeat the last chunk
    const u32x4 gdir = *reinterpret_cast<const u32x4*>(lds + goff + qd * 16);
    __syncthreads();
    // rows 1.. -> demb[b] (contiguous, non-temporal: nothing reads them before the update,
    // after the rest of the backward has passed through the caches), row 0 -> dx0[b] =
    // G[0:D) + dV_0; 16-byte stores.
    // Every thread issues a fixed number of stores (threads past the end repeat the last
    // chunk with the same bytes), so that waiting for the next sample's loads never has to
    // wait for these stores as well.
    const int nv = D * GSZ / 16;
    const int nchunk = (V - 1) * nv;
    char* derow = reinterpret_cast<char*>(demb + static_cast<int64_t>(b) * F * D);
#pragma unroll
    for (int k = 0; k < UPT * GSZ; ++k) {
      int q = k * 256 + tid;
      q = q < nchunk ? q : nchunk - 1;
      const int row = q / nv + 1, c = q - (row - 1) * nv;
      __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(lds + ooff + row * opitch + c * 16),
                                  reinterpret_cast<u32x4*>(derow + static_cast<int64_t>(q) * 16));
    }
    {
      // dx0 chunk qd = G[0:D) chunk (registers) + dV_0 chunk (fp32 in LDS; its next writer
      // runs only after the next sample's first barrier, which every thread reaches after
      // this read).  Threads past D/8 store the last chunk again with the same bytes.
      float f[8];
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const uint32_t w = gdir[x >> 1];
        const uint16_t gv = static_cast<uint16_t>((x & 1) ? (w >> 16) : (w & 0xffffu));
        f[x] = reinterpret_cast<const float*>(lds + r0off)[qd * 8 + x] + IT::to_f(gv);
      }
      store_n<GT, 8>(dx0 + static_cast<int64_t>(b) * D + qd * 8, f);
    }
  };

  int b = blockIdx.x;
  if (b >= B) return;
  if constexpr (DS) {  // S's diagonal and padding are never written: zero once
    for (int o = tid * 16; o < VP * spitch; o += 256 * 16)
      *reinterpret_cast<u32x4*>(lds + soff + o) = u32x4{0, 0, 0, 0};
    __syncthreads();
  }
  // Prologue loads land before the loop (settle), so that the wait counts the compiler
  // derives for the loop are those of its steady state alone.
  if constexpr (GATHER) {
    // Fill the pipeline synchronously: buffers 0 and 1 with samples b and b + NG, parity 0's
    // and 1's indices with b + 2 NG and b + 3 NG, their bounds with b + 4 NG and b + 5 NG --
    // the state a trip of the loop leaves for the next.
#pragma unroll
    for (int uu = 0; uu < GU; ++uu)
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int tt = row_table(uu, m);
        const int tc = tt < 0 ? 0 : tt;
        tb[uu][m] = static_cast<uint32_t>(gs.row_off[tc]);
        tr[uu][m] = static_cast<uint32_t>(gs.row_off[tc + 1] - gs.row_off[tc]);
      }
    g_bounds(b, Buf<0>{});
    g_first(Buf<0>{});
    fetch(b, Buf<0>{});
    g_bounds(b + NG, Buf<1>{});
    g_first(Buf<1>{});
    fetch(min(b + NG, B - 1), Buf<1>{});
    g_bounds(b + 2 * NG, Buf<0>{});
    g_first(Buf<0>{});
    g_bounds(b + 3 * NG, Buf<1>{});
    g_first(Buf<1>{});
    g_bounds(b + 4 * NG, Buf<0>{});
    g_bounds(b + 5 * NG, Buf<1>{});
#pragma unroll
    for (int uu = 0; uu < GU; ++uu)
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        settle_i(bnd_s[0][uu][m]); settle_i(bnd_e[0][uu][m]);
        settle_i(bnd_s[1][uu][m]); settle_i(bnd_e[1][uu][m]);
        settle_i(gix[0][uu][m]); settle_i(gix[1][uu][m]);
      }
  } else {
    fetch(b, Buf<0>{});
    if constexpr (PD == 2) fetch(min(b + NG, B - 1), Buf<1>{});
  }
  settle_buf(Buf<0>{});
  if constexpr (PD == 2) settle_buf(Buf<1>{});
  for (;;) {
    sample(b, Buf<0>{});
    b += NG;
    if (b >= B) break;
    if constexpr (PD == 2) {
      sample(b, Buf<1>{});
      b += NG;
      if (b >= B) break;
    }
  }
}

// ---------------------------------------------------------------------------------------
// fp32 FMA path (any dtypes): one wavefront per sample, vectors staged as fp32 in LDS.
// ---------------------------------------------------------------------------------------
template <class IT>
__device__ inline void stage_tile_f32(const typename IT::S* __restrict__ x0,
                                      const typename IT::S* __restrict__ emb, int b, int F, int D,
                                      float* lv) {
  const int V = F + 1;
  for (int q = threadIdx.x; q < V * D; q += 64) {
    const int row = q / D, d = q - row * D;
    const typename IT::S v = row == 0 ? x0[static_cast<int64_t>(b) * D + d]
                                      : emb[(static_cast<int64_t>(b) * F + row - 1) * D + d];
    lv[q] = IT::to_f(v);
  }
}

template <class IT, class OT>
__global__ __launch_bounds__(64) void k_dot_fwd_valu(const typename IT::S* __restrict__ x0,
                                                     const typename IT::S* __restrict__ emb, int B,
                                                     int F, int D, typename OT::S* __restrict__ out,
                                                     int out_stride) {
  extern __shared__ uint4 smem[];
  float* lv = reinterpret_cast<float*>(smem);
  const int V = F + 1;
  const int64_t P = static_cast<int64_t>(V) * (V - 1) / 2;
  for (int b = blockIdx.x; b < B; b += gridDim.x) {
    stage_tile_f32<IT>(x0, emb, b, F, D, lv);
    __syncthreads();
    typename OT::S* orow = out + static_cast<int64_t>(b) * out_stride;
    for (int d = threadIdx.x; d < D; d += 64) orow[d] = OT::from_f(lv[d]);
    // walk pairs in row-major order; lane p handles pairs p, p+64, ...
    int i = 1, j = 0;
    int64_t p = 0;
    for (int64_t target = threadIdx.x; target < P; target += 64) {
      while (p < target) {  // advance (i, j) to pair number `target`
        ++p;
        if (++j == i) { ++i; j = 0; }
      }
      float s = 0.0f;
      for (int d = 0; d < D; ++d) s = fmaf(lv[i * D + d], lv[j * D + d], s);
      orow[D + p] = OT::from_f(s);
    }
    for (int64_t c = D + P + threadIdx.x; c < out_stride; c += 64) orow[c] = OT::from_f(0.0f);
    __syncthreads();
  }
}

template <class IT, class DT, class GT>
__global__ __launch_bounds__(64) void k_dot_bwd_valu(const typename IT::S* __restrict__ x0,
                                                     const typename IT::S* __restrict__ emb, int B,
                                                     int F, int D, const typename DT::S* __restrict__ dout,
                                                     int out_stride, typename GT::S* __restrict__ dx0,
                                                     typename GT::S* __restrict__ demb) {
  extern __shared__ uint4 smem[];
  float* lv = reinterpret_cast<float*>(smem);
  const int V = F + 1;
  const int64_t P = static_cast<int64_t>(V) * (V - 1) / 2;
  float* G = lv + V * D;
  for (int b = blockIdx.x; b < B; b += gridDim.x) {
    stage_tile_f32<IT>(x0, emb, b, F, D, lv);
    const typename DT::S* grow = dout + static_cast<int64_t>(b) * out_stride;
    for (int64_t c = threadIdx.x; c < D + P; c += 64) G[c] = DT::to_f(grow[c]);
    __syncthreads();
    for (int q = threadIdx.x; q < V * D; q += 64) {
      const int k = q / D, d = q - k * D;
      float acc = 0.0f;
      for (int j = 0; j < V; ++j) {
        if (j == k) continue;
        const int hi = j > k ? j : k, lo = j > k ? k : j;
        acc = fmaf(G[D + pair_pos(hi, lo)], lv[j * D + d], acc);
      }
      if (k == 0)
        dx0[static_cast<int64_t>(b) * D + d] = GT::from_f(G[d] + acc);
      else
        demb[(static_cast<int64_t>(b) * F + k - 1) * D + d] = GT::from_f(acc);
    }
    __syncthreads();
  }
}

constexpr size_t kMaxLds = 64 * 1024;

int grid_for(int B, size_t lds_bytes) {
  // enough one-wave workgroups to fill 256 CUs several times over; each loops over samples
  const int per_cu = lds_bytes ? static_cast<int>(std::min<size_t>(16, (160 * 1024) / lds_bytes)) : 16;
  const int g = 256 * (per_cu > 0 ? per_cu : 1);
  return B < g ? B : g;
}

template <class IT, class OT, int NQ, int SPL, int WPB>
el_status launch_fwd_w(const void* x0, const void* emb, int B, int F, int D, void* out,
                       int out_stride, size_t wave_lds, hipStream_t stream) {
  const int vec_out = (static_cast<int64_t>(out_stride) * sizeof(typename OT::S)) % 16 == 0;
  auto kern = k_dot_fwd_mfma<IT, OT, NQ, SPL, WPB>;
  const int blocks = resident_grid(reinterpret_cast<const void*>(kern), (B + WPB - 1) / WPB,
                                   WPB * wave_lds, 64 * WPB);
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(64 * WPB), WPB * wave_lds, stream,
                     static_cast<const uint16_t*>(x0), static_cast<const uint16_t*>(emb), B, F, D,
                     static_cast<typename OT::S*>(out), out_stride, vec_out, static_cast<int>(wave_lds));
  return check_launch("dot_interact_fwd");
}

// Up to 4 wavefronts per workgroup, as many as fit in 64 KB of LDS.
template <class IT, class OT, int NQ, int SPL>
el_status launch_fwd_t(const void* x0, const void* emb, int B, int F, int D, void* out,
                       int out_stride, size_t lds, hipStream_t stream) {
  const size_t wave_lds = (lds + 15) / 16 * 16;
  if (4 * wave_lds <= kMaxLds)
    return launch_fwd_w<IT, OT, NQ, SPL, 4>(x0, emb, B, F, D, out, out_stride, wave_lds, stream);
  if (2 * wave_lds <= kMaxLds)
    return launch_fwd_w<IT, OT, NQ, SPL, 2>(x0, emb, B, F, D, out, out_stride, wave_lds, stream);
  return launch_fwd_w<IT, OT, NQ, SPL, 1>(x0, emb, B, F, D, out, out_stride, wave_lds, stream);
}

// Shape classes of the MFMA forward: input chunks per lane (NQ) and output-row chunks per
// lane (SPL; 0 = a loop of run-time length).
template <class IT, class OT, int NQ>
el_status launch_fwd_wide_t(const void* x0, const void* emb, int B, int F, int D, void* out,
                            int out_stride, size_t lds, hipStream_t stream) {
  auto kern = k_dot_fwd_wide<IT, OT, NQ>;
  hipLaunchKernelGGL(kern, dim3(resident_grid(reinterpret_cast<const void*>(kern), B, lds, 256)), dim3(256),
                     lds, stream, static_cast<const uint16_t*>(x0), static_cast<const uint16_t*>(emb), B, F, D,
                     static_cast<typename OT::S*>(out), out_stride);
  return check_launch("dot_interact_fwd");
}

template <class IT, class OT>
el_status launch_fwd_mfma(const void* x0, const void* emb, int B, int F, int D, void* out,
                          int out_stride, size_t lds, hipStream_t stream) {
  const int chunks = (F + 1) * (D / 8);
  if (F + 1 > 32) {  // several 32-row tiles: four wavefronts per sample, no staged output row
    const size_t tlds = static_cast<size_t>(F + 1) * (D * 2 + 16) + 16;
    if (tlds <= kMaxLds) {
      if (chunks <= 2 * 256) return launch_fwd_wide_t<IT, OT, 2>(x0, emb, B, F, D, out, out_stride, tlds, stream);
      if (chunks <= 4 * 256) return launch_fwd_wide_t<IT, OT, 4>(x0, emb, B, F, D, out, out_stride, tlds, stream);
      if (chunks <= 8 * 256) return launch_fwd_wide_t<IT, OT, 8>(x0, emb, B, F, D, out, out_stride, tlds, stream);
    }
  }
  const int64_t ochunks = (static_cast<int64_t>(out_stride) * sizeof(typename OT::S) + 15) / 16;
  if (chunks <= 8 * 64) {
    if (ochunks <= 64) return launch_fwd_t<IT, OT, 8, 1>(x0, emb, B, F, D, out, out_stride, lds, stream);
    if (ochunks <= 4 * 64) return launch_fwd_t<IT, OT, 8, 4>(x0, emb, B, F, D, out, out_stride, lds, stream);
    return launch_fwd_t<IT, OT, 8, 0>(x0, emb, B, F, D, out, out_stride, lds, stream);
  }
  if (chunks <= 16 * 64) {
    if (ochunks <= 16 * 64) return launch_fwd_t<IT, OT, 16, 16>(x0, emb, B, F, D, out, out_stride, lds, stream);
    return launch_fwd_t<IT, OT, 16, 0>(x0, emb, B, F, D, out, out_stride, lds, stream);
  }
  return launch_fwd_t<IT, OT, 32, 0>(x0, emb, B, F, D, out, out_stride, lds, stream);
}

template <class IT, class OT>
el_status fwd_typed(const void* x0, const void* emb, int B, int F, int D, void* out, int out_stride,
                    hipStream_t stream) {
  const int V = F + 1;
  if constexpr (sizeof(typename IT::S) == 2) {
    const size_t ost = (static_cast<size_t>(out_stride) * sizeof(typename OT::S) + 15) / 16 * 16;
    const size_t lds = static_cast<size_t>(V) * (D * 2 + 16) + ost + 16;
    const int chunks = V * (D / 8);
    if (D % 16 == 0 && V <= 128 && lds <= kMaxLds && chunks <= 32 * 64) {
      return launch_fwd_mfma<IT, OT>(x0, emb, B, F, D, out, out_stride, lds, stream);
    }
  }
  const size_t lds = static_cast<size_t>(V) * D * 4;
  if (lds > kMaxLds)
    return set_error(EL_ERR_UNSUPPORTED, "dot_interact_fwd: (F+1)*D too large for one LDS tile");
  hipLaunchKernelGGL((k_dot_fwd_valu<IT, OT>), dim3(grid_for(B, lds)), dim3(64), lds, stream,
                     static_cast<const typename IT::S*>(x0), static_cast<const typename IT::S*>(emb),
                     B, F, D, static_cast<typename OT::S*>(out), out_stride);
  return check_launch("dot_interact_fwd");
}

template <class IT, class GT, int UPT, int GPT, int KSM, int PD>
el_status launch_bwd_t(const void* x0, const void* emb, int B, int F, int D, const void* dout,
                       int out_stride, void* dx0, void* demb, size_t lds, hipStream_t stream) {
  auto kern = k_dot_bwd_mfma<IT, GT, UPT, GPT, KSM, PD, IT, false>;
  // up to four times the workgroups that fit at once, while each still loops over 16 samples
  // or more: workgroups that start late or run slow then hand their share to the dispatcher
  // instead of holding up the end (alone 210 -> 199 us on the training step's shape, 64 ->
  // 16 samples each; 2x: 202, 8x: 200; the multi-hot shape at 8 samples each: 166 -> 171)
  const int64_t resident = resident_grid(reinterpret_cast<const void*>(kern), B, lds, 256);
  const int64_t mul = std::max<int64_t>(1, std::min<int64_t>(4, B / (16 * resident)));
  const int64_t grid = std::min<int64_t>(B, mul * resident);
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)),
                     dim3(256), lds, stream, static_cast<const uint16_t*>(x0),
                     static_cast<const uint16_t*>(emb), B, F, D, static_cast<const uint16_t*>(dout),
                     out_stride, static_cast<typename GT::S*>(dx0), static_cast<typename GT::S*>(demb),
                     GatherSrc{});
  return check_launch("dot_interact_bwd");
}

// LDS bytes of the MFMA backward: V^T [D][VP] (pitch 2 VP + 16) | gradient row | VP x D
// output block | dV_0 in fp32 | scratch slot.
size_t bwd_lds_bytes(int F, int D, size_t gsz) {
  const int V = F + 1;
  const int64_t P = static_cast<int64_t>(V) * (V - 1) / 2;
  const int64_t gchunks = (D + P + 7) / 8;
  const size_t VP = static_cast<size_t>((V + 31) / 32 * 32);
  return static_cast<size_t>(D) * (VP * 2 + 16) + gchunks * 16 + VP * (D * gsz + 16) +
         static_cast<size_t>(D) * 4 + 16;
}

// LDS bytes of the dense-S class (gradient row in registers): V^T | dx0's direct term (D
// elements) | S [VP][VP] (pitch 2 VP + 16) | output block | dV_0 in fp32 | scratch slot.
// Two workgroups per CU of up to kMaxLdsDense bytes fit the 160 KB of LDS.
constexpr size_t kMaxLdsDense = 80 * 1024;
size_t bwd_lds_bytes_dense(int F, int D, size_t gsz) {
  const size_t VP = static_cast<size_t>((F + 1 + 31) / 32 * 32);
  return static_cast<size_t>(D) * (VP * 2 + 16) + static_cast<size_t>(D) * 2 + VP * (VP * 2 + 16) +
         VP * (D * gsz + 16) + static_cast<size_t>(D) * 4 + 16;
}

template <class TT, class IT, class GT>
el_status launch_emb_dot_bwd_t(const el_tables& tab, const el_bags& bags, uint32_t flags,
                               const void* x0, const void* dout, int out_stride, void* dx0,
                               void* demb, hipStream_t stream) {
  const int B = bags.batch, F = tab.num_tables, D = tab.dim;
  const int V = F + 1;
  const int64_t P = static_cast<int64_t>(V) * (V - 1) / 2;
  const size_t lds = bwd_lds_bytes(F, D, sizeof(typename GT::S));
  const int units = (V + 31) / 32 * 16 * (D / 8);
  if (!(D % 16 == 0 && D >= 32 && V <= 32 && units <= 256 && (D + P + 7) / 8 <= 256 &&
        out_stride % 8 == 0 && lds <= kMaxLds && bags.nnz > 0 && tab.total_rows > 0))
    return set_error(EL_ERR_UNSUPPORTED,
                     "emb_dot_bwd: the fused kernel covers 16-bit activations, D % 16 == 0, D >= 32, "
                     "F <= 31, (F+1)/2 * D/8 <= 256, out_stride % 8 == 0 and nnz > 0");
  auto kern = k_dot_bwd_mfma<IT, GT, 1, 1, 2, 2, TT, true>;
  GatherSrc gs{tab.base, tab.row_offset, bags.indices, bags.offsets, static_cast<int32_t>(bags.nnz),
               (flags & EL_FLAG_HASH_INDICES) ? 1u : 0u};
  hipLaunchKernelGGL(kern, dim3(resident_grid(reinterpret_cast<const void*>(kern), B, lds, 256)),
                     dim3(256), lds, stream, static_cast<const uint16_t*>(x0), nullptr, B, F, D,
                     static_cast<const uint16_t*>(dout), out_stride,
                     static_cast<typename GT::S*>(dx0), static_cast<typename GT::S*>(demb), gs);
  return check_launch("emb_dot_bwd");
}

// Shape classes of the MFMA backward: K steps (vectors per sample), row pairs per thread,
// gradient-row chunks per thread.  EL_ERR_UNSUPPORTED for shapes outside them.
template <class IT, class GT>
el_status launch_bwd_mfma(const void* x0, const void* emb, int B, int F, int D, const void* dout,
                          int out_stride, void* dx0, void* demb, size_t lds, hipStream_t stream) {
  const int V = F + 1;
  const int VP = (V + 31) / 32 * 32;
  const int units = VP / 2 * (D / 8);
  const int gchunks = (D + V * (V - 1) / 2 + 7) / 8;
  if (V <= 32) {
    if (units <= 256 && gchunks <= 256)
      return launch_bwd_t<IT, GT, 1, 1, 2, 2>(x0, emb, B, F, D, dout, out_stride, dx0, demb, lds, stream);
    if (units <= 512 && gchunks <= 512)
      return launch_bwd_t<IT, GT, 2, 2, 2, 1>(x0, emb, B, F, D, dout, out_stride, dx0, demb, lds, stream);
  } else if (V <= 64) {
    if (units <= 512) return launch_bwd_t<IT, GT, 2, 0, 4, 1>(x0, emb, B, F, D, dout, out_stride, dx0, demb, lds, stream);
    if (units <= 1024) return launch_bwd_t<IT, GT, 4, 0, 4, 1>(x0, emb, B, F, D, dout, out_stride, dx0, demb, lds, stream);
  } else if (V <= 128) {
    if (units <= 512 && gchunks <= 768) {
      const size_t dlds = bwd_lds_bytes_dense(F, D, sizeof(typename GT::S));
      if (dlds <= kMaxLdsDense)
        return launch_bwd_t<IT, GT, 2, 3, 8, 1>(x0, emb, B, F, D, dout, out_stride, dx0, demb, dlds, stream);
    }
    if (units <= 512) return launch_bwd_t<IT, GT, 2, 0, 8, 1>(x0, emb, B, F, D, dout, out_stride, dx0, demb, lds, stream);
    if (units <= 1024) return launch_bwd_t<IT, GT, 4, 0, 8, 1>(x0, emb, B, F, D, dout, out_stride, dx0, demb, lds, stream);
  }
  return EL_ERR_UNSUPPORTED;
}

template <class IT, class DT, class GT>
el_status bwd_typed(const void* x0, const void* emb, int B, int F, int D, const void* dout,
                    int out_stride, void* dx0, void* demb, hipStream_t stream) {
  const int V = F + 1;
  const int64_t P = static_cast<int64_t>(V) * (V - 1) / 2;
  if constexpr (sizeof(typename IT::S) == 2 && IT::code == DT::code) {
    const size_t lds = bwd_lds_bytes(F, D, sizeof(typename GT::S));
    // 16-byte chunks of the gradient row must stay inside the row: stride multiple of 8
    // D = 16: the fp32 FMA kernel (one wavefront per sample) is faster than a half-empty
    // 32-row MFMA tile driven by four wavefronts
    if (D % 16 == 0 && D >= 32 && V <= 128 && lds <= kMaxLds && out_stride % 8 == 0) {
      const el_status st = launch_bwd_mfma<IT, GT>(x0, emb, B, F, D, dout, out_stride, dx0, demb, lds, stream);
      if (st != EL_ERR_UNSUPPORTED) return st;
    }
  }
  const size_t lds = (static_cast<size_t>(V) * D + D + P) * 4;
  if (lds > kMaxLds)
    return set_error(EL_ERR_UNSUPPORTED, "dot_interact_bwd: (F+1)*D + pairs too large for LDS");
  hipLaunchKernelGGL((k_dot_bwd_valu<IT, DT, GT>), dim3(grid_for(B, lds)), dim3(64), lds, stream,
                     static_cast<const typename IT::S*>(x0), static_cast<const typename IT::S*>(emb),
                     B, F, D, static_cast<const typename DT::S*>(dout), out_stride,
                     static_cast<typename GT::S*>(dx0), static_cast<typename GT::S*>(demb));
  return check_launch("dot_interact_bwd");
}

// dtype dispatch helpers
template <class F>
el_status with_type(el_dtype d, F&& f) {
  switch (d) {
    case EL_F32: return f(F32T{});
    case EL_F16: return f(F16T{});
    case EL_BF16: return f(BF16T{});
    default: break;
  }
  return set_error(EL_ERR_INVALID_ARG, "unknown dtype");
}

}  // namespace

el_status launch_dot_fwd(const void* x0, const void* emb, el_dtype in_dtype, int B, int F, int D,
                         void* out, el_dtype out_dtype, int out_stride, hipStream_t stream) {
  return with_type(in_dtype, [&](auto it) {
    return with_type(out_dtype, [&](auto ot) {
      return fwd_typed<decltype(it), decltype(ot)>(x0, emb, B, F, D, out, out_stride, stream);
    });
  });
}

el_status launch_emb_dot_bwd(const el_tables& tab, const el_bags& bags, uint32_t flags,
                             const void* x0, el_dtype act_dtype, const void* dout, int out_stride,
                             void* dx0, void* demb, el_dtype grad_dtype, hipStream_t stream) {
  if (act_dtype == EL_F32)
    return set_error(EL_ERR_UNSUPPORTED, "emb_dot_bwd: the fused kernel takes 16-bit activations");
  return with_type(tab.dtype, [&](auto tt) {
    return with_type(act_dtype, [&](auto it) {
      return with_type(grad_dtype, [&](auto gt) {
        using IT = decltype(it);
        if constexpr (sizeof(typename IT::S) == 2)
          return launch_emb_dot_bwd_t<decltype(tt), IT, decltype(gt)>(tab, bags, flags, x0, dout,
                                                                      out_stride, dx0, demb, stream);
        else
          return EL_ERR_UNSUPPORTED;
      });
    });
  });
}

el_status launch_dot_bwd(const void* x0, const void* emb, el_dtype in_dtype, int B, int F, int D,
                         const void* dout, el_dtype dout_dtype, int out_stride, void* dx0,
                         void* demb, el_dtype grad_dtype, hipStream_t stream) {
  return with_type(in_dtype, [&](auto it) {
    return with_type(dout_dtype, [&](auto dt) {
      return with_type(grad_dtype, [&](auto gt) {
        return bwd_typed<decltype(it), decltype(dt), decltype(gt)>(x0, emb, B, F, D, dout, out_stride,
                                                                   dx0, demb, stream);
      });
    });
  });
}

}  // namespace el
