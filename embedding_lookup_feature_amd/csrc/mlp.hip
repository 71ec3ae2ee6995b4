// mlp.hip -- the dense layers of the bottom and top MLPs on gfx950 MFMA, the logistic loss
// on the final logit, and plain SGD on the dense parameters.
//
// Page "DLRM For PyTorch", §Model architecture: the dense features pass through the bottom
// MLP (linear layers, each followed by a ReLU); the interaction output, concatenated with
// the bottom-MLP output, passes through the top MLP, which ends in one number read as a
// click likelihood.  §Command-line options gives the widths (--bottom_mlp_sizes 512,256,128,
// --top_mlp_sizes 1024,1024,512,256,1) and the page trains the MLPs in mixed precision:
// 16-bit operands with fp32 master weights.
//
// One tiled MFMA kernel serves the three products of a layer.  With weights w[n][k]:
//   forward   y[m][n]  = sum_k x[m][k]  w[n][k]   rows operand x  (reduction contiguous),
//                                                  cols operand w  (reduction contiguous)
//   data grad dx[m][k] = sum_n dz[m][n] w[n][k]   rows operand dz (reduction contiguous),
//                                                  cols operand w  (output contiguous)
//   weight    dw[n][k] = sum_m dz[m][n] x[m][k]   rows operand dz (output contiguous),
//                                                  cols operand x  (output contiguous)
// Both operands are staged through LDS as [row][reduction] tiles (an 8 x 8 register
// transpose for operands whose output index is the contiguous one), then read as
// v_mfma_f32_32x32x16 fragments.  The MFMA "A" operand is the cols operand, so each lane's
// accumulator registers hold 4 consecutive output columns of one output row: the epilogue
// stores 8 (16-bit) or 16 (fp32) contiguous bytes per lane.
#include <algorithm>
#include <cstdio>
#include <string>

#include "el_internal.hpp"
#include "el_mfma.hpp"

namespace el {
namespace {

constexpr int kBK = 64;           // reduction per LDS stage
constexpr int kPitch = kBK + 8;   // LDS row pitch in elements (144 B: 16-B reads conflict-free)

// Tile shapes: WR x WC wavefronts, each owning FR x FC tiles of 32 x 32 outputs (FR along
// output rows, FC along output columns); BR x BC outputs per workgroup.
template <int WR_, int WC_, int FR_, int FC_>
struct Cfg {
  static constexpr int WR = WR_, WC = WC_, FR = FR_, FC = FC_;
  static constexpr int BR = WR * FR * 32, BC = WC * FC * 32;
  static constexpr int NT = WR * WC * 64;
  static constexpr int WPS = NT == 256 ? 2 : 1;  // workgroups per CU the kernel is built for
};
using CfgS = Cfg<2, 2, 2, 2>;  // 128 x 128 outputs, 256 threads, two workgroups per CU
using CfgL = Cfg<2, 4, 4, 2>;  // 256 x 256 outputs, 512 threads, wavefront 128 x 64, one per CU

enum Epi { EPI_FWD = 0, EPI_DGRAD = 1, EPI_WGRAD = 2 };

struct GemmArgs {
  const uint16_t* P;  // rows operand
  long ldp;
  const uint16_t* Q;  // cols operand
  long ldq;
  int R, C;           // output rows, cols
  int red;            // reduction length
  int red_per_split;  // reduction per split (multiple of kBK)
  int tiles_c, tiles;  // column tiles, tiles per split
  void* out;          // fwd / dgrad: [R][ldo] 16-bit; wgrad: fp32 [split][R][ldo]
  long ldo;
  long split_stride;  // wgrad: elements between the partial planes of two splits
  const float* bias;  // fwd: [C] or null
  int relu;           // fwd: ReLU; dgrad: multiply by 1[mask > 0]
  const uint16_t* mask;  // dgrad: [R][ldm]
  long ldm;
  float* dbp;         // wgrad: [split][R] row sums of the rows operand (bias gradient)
};

// 16 bytes from global memory.  The load is unconditional (from `safe`, the operand's base,
// for a vector outside the operand) so that no branch splits the stream of loads; the caller
// zeroes such vectors only when it writes them to LDS, so nothing waits for a load before
// its stage needs it.
__device__ inline u32x4 ld16(const uint16_t* p, const uint16_t* safe, bool ok) {
  return *reinterpret_cast<const u32x4*>(ok ? p : safe);
}
__device__ inline u32x4 keep_if(const u32x4& v, uint32_t mask, int i) {
  return ((mask >> i) & 1u) ? v : u32x4{0, 0, 0, 0};
}

// Global -> registers for one reduction-contiguous operand tile of ROWS rows x 64
// reduction; NT threads, ROWS*8/NT vectors each (thread t: row t/8 + (NT/8) i, reduction
// 8 (t%8) .. +8).
// FULL: every vector of every computed stage lies inside the operand (the grid's tiles are
// whole and the stage count is even), so no vector is masked; the loads the pipeline issues
// ahead for stages past the last are pointed at the last stage (see k_at in k_gemm).
template <int ROWS, int NT, bool FULL>
struct TileLoaderRC {
  static constexpr int N = ROWS * 8 / NT;
  u32x4 v[N];
  uint32_t ok = 0;  // bit i: vector i lies inside the operand
  __device__ inline void load(const uint16_t* base, long ld, int row0, int nrows, int k0, int kend,
                              int sub) {
    const int kk = k0 + (sub & 7) * 8;
    ok = 0;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int r = row0 + (sub >> 3) + (NT / 8) * i;
      if constexpr (FULL) {
        v[i] = *reinterpret_cast<const u32x4*>(base + static_cast<long>(r) * ld + kk);
      } else {
        const bool in = r < nrows && kk < kend;
        v[i] = ld16(base + static_cast<long>(r) * ld + kk, base, in);
        ok |= static_cast<uint32_t>(in) << i;
      }
    }
  }
  __device__ inline void store(uint16_t* lds, int sub) const {
#pragma unroll
    for (int i = 0; i < N; ++i)
      *reinterpret_cast<u32x4*>(lds + ((sub >> 3) + (NT / 8) * i) * kPitch + (sub & 7) * 8) =
          FULL ? v[i] : keep_if(v[i], ok, i);
  }
};

// Both operands output-contiguous (the weight gradient, global [red][rows]): threads
// 0..BR-1 fetch the rows operand's BR blocks of 8 rows x 8 reductions and threads
// BR..BR+BC-1 the cols operand's, through one code path (operand chosen by per-thread
// selects, no branch between the two sets of loads); each block is transposed in
// registers on its way to LDS.
template <int BR, bool FULL>
struct PairLoaderOC {
  u32x4 v[8];
  uint32_t ok = 0;
  const uint16_t* base;
  long ld;
  int row0, nrows, sub;
  __device__ inline PairLoaderOC(const GemmArgs& a, int tid, int prow0, int qcol0) {
    const bool q = tid >= BR;
    base = q ? a.Q : a.P;
    ld = q ? a.ldq : a.ldp;
    row0 = q ? qcol0 : prow0;
    nrows = q ? a.C : a.R;
    sub = q ? tid - BR : tid;
  }
  __device__ inline void load(int k0, int kend) {
    const int kb = sub & 7, rb = sub >> 3;
    const int r = row0 + rb * 8;
    ok = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = k0 + kb * 8 + i;
      if constexpr (FULL) {
        v[i] = *reinterpret_cast<const u32x4*>(base + static_cast<long>(k) * ld + r);
      } else {
        const bool in = r < nrows && k < kend;
        v[i] = ld16(base + static_cast<long>(k) * ld + r, base, in);
        ok |= static_cast<uint32_t>(in) << i;
      }
    }
  }
  __device__ inline void store(uint16_t* lds) const {
    const int kb = sub & 7, rb = sub >> 3;
    u32x4 z[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] = FULL ? v[i] : keep_if(v[i], ok, i);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int w = j >> 1;
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t a = z[2 * q][w], b = z[2 * q + 1][w];
        o[q] = (j & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
      }
      *reinterpret_cast<u32x4*>(lds + (rb * 8 + j) * kPitch + kb * 8) = o;
    }
  }
};

// One LDS stage of the product: this wavefront's (FR*32) x (FC*32) block accumulates the
// kBK-long slice held in P (rows operand) and Q (cols operand); with DB, threads 0..BR-1
// also add up their row of P (the bias gradient of the weight-gradient launch).
template <class T, class C, bool DB>
__device__ __forceinline__ void gemm_stage(const uint16_t* P, const uint16_t* Q, int wr, int wc, int half,
                                           int l32, f32x16 (&acc)[C::FC][C::FR], bool do_db, int tid,
                                           float& dbsum) {
#pragma unroll
  for (int ks = 0; ks < kBK / 16; ++ks) {
    const int ko = ks * 16 + half * 8;
    u32x4 qa[C::FC], pb[C::FR];
#pragma unroll
    for (int i = 0; i < C::FC; ++i)
      qa[i] = *reinterpret_cast<const u32x4*>(Q + (wc * C::FC * 32 + i * 32 + l32) * kPitch + ko);
#pragma unroll
    for (int j = 0; j < C::FR; ++j)
      pb[j] = *reinterpret_cast<const u32x4*>(P + (wr * C::FR * 32 + j * 32 + l32) * kPitch + ko);
#pragma unroll
    for (int i = 0; i < C::FC; ++i)
#pragma unroll
      for (int j = 0; j < C::FR; ++j) acc[i][j] = mfma32<T>(qa[i], pb[j], acc[i][j]);
  }
  if (DB && do_db) {
    const uint16_t* row = P + tid * kPitch;
#pragma unroll
    for (int v = 0; v < kBK / 8; ++v) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(row + v * 8);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        dbsum += T::to_f(static_cast<uint16_t>(x[q] & 0xffffu)) + T::to_f(static_cast<uint16_t>(x[q] >> 16));
    }
  }
}

template <class T, class C, bool P_RC, bool Q_RC, int EPI, bool FULL>
__global__ __launch_bounds__(C::NT, C::WPS) void k_gemm(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sP[2][C::BR * kPitch];
  __shared__ __attribute__((aligned(16))) uint16_t sQ[2][C::BC * kPitch];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // One flat grid of tiles x splits, in split-major logical order, handed to the XCDs in
  // contiguous runs: the workgroups of one split (which share its batch slice of both
  // operands) and the neighbouring tiles of one output row (which share a panel) meet in
  // the same L2.
  const int nb = static_cast<int>(gridDim.x);
  const int lid = (nb & 7) == 0 ? xcd_remap(blockIdx.x, nb) : static_cast<int>(blockIdx.x);
  const int split = lid / a.tiles;
  const int bid = lid - split * a.tiles;
  const int tr = bid / a.tiles_c, tc = bid - tr * a.tiles_c;
  const int row0 = tr * C::BR, col0 = tc * C::BC;
  const int kbeg = split * a.red_per_split;
  const int kend = min(a.red, kbeg + a.red_per_split);
  const int nk = (kend - kbeg + kBK - 1) / kBK;

  const int wr = wave / C::WC, wc = wave % C::WC;  // this wavefront's block of the tile
  const int half = lane >> 5, l32 = lane & 31;
  f32x16 acc[C::FC][C::FR];
#pragma unroll
  for (int i = 0; i < C::FC; ++i)
#pragma unroll
    for (int j = 0; j < C::FR; ++j) acc[i][j] = f32x16{};

  // bias gradient (weight-gradient launch): the first column tile sums its rows operand
  const bool do_db = (EPI == EPI_WGRAD) && tc == 0 && tid < C::BR;
  float dbsum = 0.f;

  // Two register sets, stage t's tile in set t % 2, and two LDS buffers.  Stage kt writes
  // tile kt+1 (its loads issued two stages earlier) into the LDS buffer stage kt-1 has
  // finished with, issues the loads of tile kt+3 into the set just written out, then
  // multiplies tile kt: every load has two stages of products to arrive.  The stage count is
  // rounded up to even; stages past the reduction load zeros (masked, from the operand's
  // base), so the loop body has no branch and the compiler waits for exactly the older set.
  // The last two iterations also issue loads for up to three stages that are never
  // multiplied: unmasked (FULL), those re-read the last stage, so that no load leaves the
  // operand.  Scheduling fences keep each stage's LDS writes after the previous barrier and
  // its loads ahead of its products, so no wait for a newer set is pulled into a stage.
  const int nk2 = (nk + 1) & ~1;
  auto k_at = [&](int t) { return kbeg + (FULL && t >= nk ? nk - 1 : t) * kBK; };
  if constexpr (P_RC && Q_RC) {
    TileLoaderRC<C::BR, C::NT, FULL> pA;
    TileLoaderRC<C::BC, C::NT, FULL> qA;
    pA.load(a.P, a.ldp, row0, a.R, k_at(0), kend, tid);
    qA.load(a.Q, a.ldq, col0, a.C, k_at(0), kend, tid);
    pA.store(sP[0], tid);
    qA.store(sQ[0], tid);
    pA.load(a.P, a.ldp, row0, a.R, k_at(1), kend, tid);
    qA.load(a.Q, a.ldq, col0, a.C, k_at(1), kend, tid);
    __syncthreads();
    for (int kt = 0; kt < nk2; kt += 2) {
      __builtin_amdgcn_sched_barrier(0);
      pA.store(sP[1], tid);
      qA.store(sQ[1], tid);
      pA.load(a.P, a.ldp, row0, a.R, k_at(kt + 2), kend, tid);
      qA.load(a.Q, a.ldq, col0, a.C, k_at(kt + 2), kend, tid);
      __builtin_amdgcn_sched_barrier(0);
      gemm_stage<T, C, false>(sP[0], sQ[0], wr, wc, half, l32, acc, false, tid, dbsum);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      pA.store(sP[0], tid);
      qA.store(sQ[0], tid);
      pA.load(a.P, a.ldp, row0, a.R, k_at(kt + 3), kend, tid);
      qA.load(a.Q, a.ldq, col0, a.C, k_at(kt + 3), kend, tid);
      __builtin_amdgcn_sched_barrier(0);
      gemm_stage<T, C, false>(sP[1], sQ[1], wr, wc, half, l32, acc, false, tid, dbsum);
      __syncthreads();
    }
  } else {
    static_assert(!P_RC && !Q_RC, "mixed operand layouts are not instantiated");
    static_assert(C::BR + C::BC == C::NT, "one 8 x 8 block per thread");
    PairLoaderOC<C::BR, FULL> lA(a, tid, row0, col0);
    uint16_t* dst0 = tid >= C::BR ? sQ[0] : sP[0];
    uint16_t* dst1 = tid >= C::BR ? sQ[1] : sP[1];
    lA.load(k_at(0), kend);
    lA.store(dst0);
    lA.load(k_at(1), kend);
    __syncthreads();
    for (int kt = 0; kt < nk2; kt += 2) {
      __builtin_amdgcn_sched_barrier(0);
      lA.store(dst1);
      lA.load(k_at(kt + 2), kend);
      __builtin_amdgcn_sched_barrier(0);
      gemm_stage<T, C, EPI == EPI_WGRAD>(sP[0], sQ[0], wr, wc, half, l32, acc, do_db, tid, dbsum);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      lA.store(dst0);
      lA.load(k_at(kt + 3), kend);
      __builtin_amdgcn_sched_barrier(0);
      gemm_stage<T, C, EPI == EPI_WGRAD>(sP[1], sQ[1], wr, wc, half, l32, acc, do_db, tid, dbsum);
      __syncthreads();
    }
  }

  if (EPI == EPI_WGRAD && do_db && row0 + tid < a.R) a.dbp[static_cast<long>(split) * a.R + row0 + tid] = dbsum;

  // Epilogue: register rr of acc[i][j] is output column col0 + wc*FC*32 + i*32 + 8(rr/4) +
  // 4 half + rr%4 of output row row0 + wr*FR*32 + j*32 + l32.
#pragma unroll
  for (int j = 0; j < C::FR; ++j) {
    const int r = row0 + wr * C::FR * 32 + j * 32 + l32;
    if (r >= a.R) continue;
#pragma unroll
    for (int i = 0; i < C::FC; ++i) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = col0 + wc * C::FC * 32 + i * 32 + g * 8 + half * 4;
        if (c >= a.C) continue;
        float v[4] = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
        if constexpr (EPI == EPI_WGRAD) {
          float* o = static_cast<float*>(a.out) + static_cast<long>(split) * a.split_stride +
                     static_cast<long>(r) * a.ldo + c;
          *reinterpret_cast<float4*>(o) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
          if constexpr (EPI == EPI_FWD) {
            if (a.bias) {
#pragma unroll
              for (int q = 0; q < 4; ++q) v[q] += a.bias[c + q];
            }
            if (a.relu) {
#pragma unroll
              for (int q = 0; q < 4; ++q) v[q] = v[q] > 0.f ? v[q] : 0.f;
            }
          } else {
            if (a.relu) {
              const uint2 m = *reinterpret_cast<const uint2*>(a.mask + static_cast<long>(r) * a.ldm + c);
              const uint32_t mw[2] = {m.x, m.y};
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const float x = T::to_f(static_cast<uint16_t>((mw[q >> 1] >> (16 * (q & 1))) & 0xffffu));
                if (!(x > 0.f)) v[q] = 0.f;
              }
            }
          }
          store_n<T, 4>(static_cast<uint16_t*>(a.out) + static_cast<long>(r) * a.ldo + c, v);
        }
      }
    }
  }
}

// wt[k][n] = w[n][k] for a [N][K] 16-bit matrix (N, K multiples of 8): one 8 x 8 block
// per thread, transposed in registers.
__global__ __launch_bounds__(256) void k_transpose16(const uint16_t* w, uint16_t* wt, int N, int K) {
  const int kv = K / 8;
  const long g = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (g >= static_cast<long>(N / 8) * kv) return;
  const int nb = static_cast<int>(g / kv), kb = static_cast<int>(g - static_cast<long>(nb) * kv);
  u32x4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    v[i] = *reinterpret_cast<const u32x4*>(w + static_cast<long>(nb * 8 + i) * K + kb * 8);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int q2 = j >> 1;
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t a = v[2 * q][q2], b = v[2 * q + 1][q2];
      o[q] = (j & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
    }
    *reinterpret_cast<u32x4*>(wt + static_cast<long>(kb * 8 + j) * N + nb * 8) = o;
  }
}

// Ordered sum of the split partials: out[c] = sum_s part[s][c] (c < n; VEC consecutive
// columns per thread, n % VEC == 0), for workgroup `blk` of the array.  Each workgroup
// covers 16 column vectors with 16 split groups: group g adds splits g, g+16, g+32, ... in
// order (loads issued 8 at a time), then the 16 group sums are added in group order.
// Bitwise reproducible.
template <int VEC>
__device__ inline void split_sum_block(const float* part, long n, int splits, float* out, long blk) {
  constexpr int SG = 16, CV = 256 / SG;
  __shared__ float red[SG][CV * VEC];
  const int t = threadIdx.x, cv = t % CV, sg = t / CV;
  const long c = (blk * CV + cv) * VEC;
  float s[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) s[e] = 0.f;
  if (c < n) {
    for (int p0 = sg; p0 < splits; p0 += SG * 8) {
      float v[8][VEC];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int p = p0 + q * SG;
        if (p < splits) {
          if constexpr (VEC == 4) {
            const float4 x = *reinterpret_cast<const float4*>(part + p * n + c);
            v[q][0] = x.x; v[q][1] = x.y; v[q][2] = x.z; v[q][3] = x.w;
          } else {
            v[q][0] = part[p * n + c];
          }
        }
      }
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (p0 + q * SG < splits) {
#pragma unroll
          for (int e = 0; e < VEC; ++e) s[e] += v[q][e];
        }
    }
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) red[sg][cv * VEC + e] = s[e];
  __syncthreads();
  if (sg == 0 && c < n) {
    float o[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) o[e] = red[0][cv * VEC + e];
    for (int g = 1; g < SG; ++g)
#pragma unroll
      for (int e = 0; e < VEC; ++e) o[e] += red[g][cv * VEC + e];
    if constexpr (VEC == 4) {
      *reinterpret_cast<float4*>(out + c) = make_float4(o[0], o[1], o[2], o[3]);
    } else {
      out[c] = o[0];
    }
  }
}

// The weight partials (4 columns per thread) in the first b4 workgroups, the bias partials
// (one per thread) in the rest: one launch for both sums of a layer's gradient.
__global__ __launch_bounds__(256) void k_split_sum(const float* part, long n, float* out, const float* dbp,
                                                   long nb, float* db, int splits, long b4) {
  if (blockIdx.x < b4)  // block-uniform
    split_sum_block<4>(part, n, splits, out, blockIdx.x);
  else
    split_sum_block<1>(dbp, nb, splits, db, blockIdx.x - b4);
}

void launch_split_sum(const float* part, long n, int splits, float* out, const float* dbp, long nb, float* db,
                      hipStream_t st) {
  const long b4 = (n / 4 + 15) / 16;
  const long b1 = (nb + 15) / 16;
  hipLaunchKernelGGL(k_split_sum, dim3(static_cast<unsigned>(b4 + b1)), dim3(256), 0, st, part, n, out, dbp, nb, db,
                     splits, b4);
}

// ---------------------------------------------------------------------------------------
// One-output layers (the logit): y[m] = act(sum_k x[m][k] w[k] + b).  A group of L lanes
// (L = power of two, 8 elements per lane and step) per row; rows per wavefront 64 / L.
// ---------------------------------------------------------------------------------------
template <class T, int L>
__global__ __launch_bounds__(256) void k_gemv_fwd(const uint16_t* x, long ldx, int M, int K,
                                                 const uint16_t* w, const float* bias, int relu,
                                                 uint16_t* y, long ldy) {
  const int lane = threadIdx.x & 63;
  const int sub = lane % L;
  const long rows_per_block = (blockDim.x / 64) * (64 / L);
  const long m = blockIdx.x * rows_per_block + (threadIdx.x / 64) * (64 / L) + lane / L;
  float s = 0.f;
  if (m < M) {
    for (int k = sub * 8; k < K; k += L * 8) {
      float xf[8], wf[8];
      unpack16<T>(*reinterpret_cast<const uint4*>(x + m * ldx + k), xf);
      unpack16<T>(*reinterpret_cast<const uint4*>(w + k), wf);
#pragma unroll
      for (int q = 0; q < 8; ++q) s += xf[q] * wf[q];
    }
  }
#pragma unroll
  for (int o = L / 2; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  if (m < M && sub == 0) {
    if (bias) s += bias[0];
    if (relu && !(s > 0.f)) s = 0.f;
    y[m * ldy] = T::from_f(s);
  }
}

// dx[m][k] = dz[m] * w[k] (times 1[x[m][k] > 0] with the mask), 8 elements per thread.
template <class T>
__global__ __launch_bounds__(256) void k_gemv_dgrad(const uint16_t* dz, long ldz, int M, int K,
                                                   const uint16_t* w, const uint16_t* mask, long ldm,
                                                   uint16_t* dx, long lddx) {
  const int kv = K / 8;
  const long g = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (g >= static_cast<long>(M) * kv) return;
  const long m = g / kv;
  const int k = static_cast<int>(g - m * kv) * 8;
  const float d = T::to_f(dz[m * ldz]);
  float wf[8], v[8];
  unpack16<T>(*reinterpret_cast<const uint4*>(w + k), wf);
#pragma unroll
  for (int q = 0; q < 8; ++q) v[q] = d * wf[q];
  if (mask) {
    float xf[8];
    unpack16<T>(*reinterpret_cast<const uint4*>(mask + m * ldm + k), xf);
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (!(xf[q] > 0.f)) v[q] = 0.f;
  }
  store_n<T, 8>(dx + m * lddx + k, v);
}

// Weight / bias gradient of a one-output layer over the rows of one split:
//   part[split][k] = sum_m dz[m] x[m][k],  dbp[split] = sum_m dz[m]
// Threads: K/8 lanes per row group, G = 256 / (K/8) row groups striding over the rows; the
// groups are combined in LDS in fixed order.
template <class T>
__global__ __launch_bounds__(256) void k_gemv_wgrad(const uint16_t* x, long ldx, int M, int K,
                                                   const uint16_t* dz, long ldz, int rows_per_split,
                                                   float* part, float* dbp) {
  __shared__ float red[256 * 8 + 256];
  const int kv = K / 8;
  const int G = 256 / kv;
  const int t = threadIdx.x, grp = t / kv, kk = (t % kv) * 8;
  const int m0 = blockIdx.x * rows_per_split;
  const int m1 = min(M, m0 + rows_per_split);
  float s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float sd = 0.f;
  if (grp < G) {
    for (int m = m0 + grp; m < m1; m += G) {
      const float d = T::to_f(dz[static_cast<long>(m) * ldz]);
      float xf[8];
      unpack16<T>(*reinterpret_cast<const uint4*>(x + static_cast<long>(m) * ldx + kk), xf);
#pragma unroll
      for (int q = 0; q < 8; ++q) s[q] += d * xf[q];
      sd += d;
    }
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) red[t * 8 + q] = s[q];
  red[256 * 8 + t] = sd;
  __syncthreads();
  if (t < kv) {
    float o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int g2 = 0; g2 < G; ++g2)
#pragma unroll
      for (int q = 0; q < 8; ++q) o[q] += red[(g2 * kv + t) * 8 + q];
#pragma unroll
    for (int q = 0; q < 8; ++q) part[static_cast<long>(blockIdx.x) * K + kk + q] = o[q];
  }
  if (t == 0) {
    float o = 0.f;
    for (int g2 = 0; g2 < G; ++g2) o += red[256 * 8 + g2 * kv];
    dbp[blockIdx.x] = o;
  }
}

// ---------------------------------------------------------------------------------------
// Logistic loss on logits z [M] with labels in {0,1}: dz[m] = (sigmoid(z_m) - y_m) / M and
// loss = (1/M) sum_m [max(z,0) - z y + log(1 + exp(-|z|))].  Workgroup w handles samples
// [256 w, 256 w + 256): one per thread, its loss terms summed in a fixed tree into
// partial[w] (double); one workgroup then adds the partials in order.  Bitwise reproducible.
// ---------------------------------------------------------------------------------------
constexpr int kBceBlock = 256;

template <class T>
__global__ __launch_bounds__(kBceBlock) void k_bce_grad(const uint16_t* z, long ldz, const float* labels, int M,
                                                       uint16_t* dz, long lddz, double* partial) {
  __shared__ double red[kBceBlock];
  const int t = threadIdx.x;
  const int m = blockIdx.x * kBceBlock + t;
  double s = 0.0;
  if (m < M) {
    const float v = T::to_f(z[static_cast<long>(m) * ldz]);
    const float y = labels[m];
    s = static_cast<double>(fmaxf(v, 0.f) - v * y + log1pf(expf(-fabsf(v))));
    const float p = 1.f / (1.f + expf(-v));
    dz[static_cast<long>(m) * lddz] = T::from_f((p - y) / static_cast<float>(M));
  }
  red[t] = s;
  __syncthreads();
  for (int o = kBceBlock / 2; o > 0; o >>= 1) {
    if (t < o) red[t] += red[t + o];
    __syncthreads();
  }
  if (t == 0) partial[blockIdx.x] = red[0];
}

__global__ __launch_bounds__(1024) void k_bce_sum(const double* partial, int nparts, int M, float* loss) {
  __shared__ double red[1024];
  const int t = threadIdx.x;
  double s = 0.0;
  for (int i = t; i < nparts; i += 1024) s += partial[i];
  red[t] = s;
  __syncthreads();
  for (int o = 512; o > 0; o >>= 1) {
    if (t < o) red[t] += red[t + o];
    __syncthreads();
  }
  if (t == 0) loss[0] = static_cast<float>(red[0] / M);
}

// dz = dy * 1[y > 0], 8 elements per thread ([M] rows of stride ld, N % 8 == 0).
template <class T>
__global__ __launch_bounds__(256) void k_relu_bwd(const uint16_t* dy, const uint16_t* y, uint16_t* dz,
                                                 int M, int N, long ld) {
  const int nv = N / 8;
  const long g = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (g >= static_cast<long>(M) * nv) return;
  const long m = g / nv;
  const long off = m * ld + (g - m * nv) * 8;
  const uint4 d = *reinterpret_cast<const uint4*>(dy + off);
  const uint4 v = *reinterpret_cast<const uint4*>(y + off);
  const uint32_t dw[4] = {d.x, d.y, d.z, d.w}, vw[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const bool lo = T::to_f(static_cast<uint16_t>(vw[q] & 0xffffu)) > 0.f;
    const bool hi = T::to_f(static_cast<uint16_t>(vw[q] >> 16)) > 0.f;
    o[q] = (lo ? (dw[q] & 0xffffu) : 0u) | (hi ? (dw[q] & 0xffff0000u) : 0u);
  }
  *reinterpret_cast<uint4*>(dz + off) = uint4{o[0], o[1], o[2], o[3]};
}

__global__ __launch_bounds__(256) void k_fill_zero(float* p, long n) {
  const long i = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

// master[i] -= lr * grad[i] (one fp32 rounding); copy[i] = master[i] in the copy's dtype.
template <class T>
__global__ __launch_bounds__(256) void k_sgd_dense(float* master, uint16_t* copy, const float* grad,
                                                  long n, float lr) {
  const long i = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float v = fmaf(-lr, grad[i], master[i]);
  master[i] = v;
  if (copy) copy[i] = T::from_f(v);
}

__global__ __launch_bounds__(256) void k_sgd_dense_f32(float* master, const float* grad, long n, float lr) {
  const long i = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  master[i] = fmaf(-lr, grad[i], master[i]);
}

// ---------------------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------------------
el_status bad(const char* fn, const std::string& what) {
  return set_error(EL_ERR_INVALID_ARG, std::string(fn) + ": " + what);
}
bool al(const void* p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

struct WgradPlan {
  bool large = false;   // 256 x 256 output tiles (else 128 x 128)
  int splits = 1;
  int per = 0;        // reduction rows per split
  size_t wt_bytes = 0;  // transposed weights for the data gradient (256-byte multiple)
  size_t bytes = 0;     // total
};

// The 256 x 256 tile halves the operand bytes each output needs from L2 and LDS, but one
// workgroup fills a CU: it is taken only when its tiles still cover the chip twice.
bool use_large(long rows, long cols) {
  const long tiles = ((rows + CfgL::BR - 1) / CfgL::BR) * ((cols + CfgL::BC - 1) / CfgL::BC);
  return tiles >= 512;
}

template <class C>
void fill_tiles(GemmArgs& a) {
  a.tiles_c = (a.C + C::BC - 1) / C::BC;
  a.tiles = ((a.R + C::BR - 1) / C::BR) * a.tiles_c;
}

// Splits of the weight-gradient reduction over the batch: enough workgroups to fill every
// CU's workgroup slots once (output tiles x splits >= 512 small or 256 large tiles), each
// split at least 8 LDS stages long (with 4, the 256 -> 128 layer's 256 splits of 256 rows
// spent more on partials and pipeline fill than they gained: its backward 62 -> 56 us at
// B = 65536 with 8).
// Large tiles once the output holds at least 8 of them (one workgroup per CU, so more
// splits; with fewer tiles the split partials outweigh what the larger tile saves).
WgradPlan plan_wgrad(int M, int K, int N) {
  WgradPlan p;
  if (M <= 0) return p;
  if (N == 1) {
    const int64_t per = std::max<int64_t>(256, (static_cast<int64_t>(M) + 1023) / 1024);
    p.splits = static_cast<int>((M + per - 1) / per);
    p.per = static_cast<int>(per);
    p.bytes = static_cast<size_t>(p.splits) * (static_cast<size_t>(K) + 1) * sizeof(float);
    return p;
  }
  // 64-bit arithmetic: the sizes may be anything up to 2^31 - 1 here
  const int64_t M64 = M, N64 = N, K64 = K;
  p.large = ((N64 + CfgL::BR - 1) / CfgL::BR) * ((K64 + CfgL::BC - 1) / CfgL::BC) >= 8;
  const int64_t br = p.large ? CfgL::BR : CfgS::BR, bc = p.large ? CfgL::BC : CfgS::BC;
  const int64_t tiles = ((N64 + br - 1) / br) * ((K64 + bc - 1) / bc);
  const int64_t target = p.large ? 256 : 512;  // workgroups: two per CU (small tiles), one (large)
  int64_t s = std::max<int64_t>(1, (target + tiles - 1) / tiles);
  const int64_t max_s = std::max<int64_t>(1, M64 / (8 * kBK));
  s = std::min<int64_t>(std::min(s, max_s), 256);
  int64_t per = (M64 + s - 1) / s;
  per = std::min<int64_t>((per + kBK - 1) / kBK * kBK, INT32_MAX / kBK * kBK);
  p.splits = static_cast<int>((M64 + per - 1) / per);
  p.per = static_cast<int>(per);
  p.wt_bytes = (static_cast<size_t>(N) * K * 2 + 255) / 256 * 256;
  p.bytes = p.wt_bytes +
            (p.splits > 1 ? static_cast<size_t>(p.splits) * (static_cast<size_t>(N) * K + N) * sizeof(float) : 0);
  return p;
}

// One product, launched with the tile configuration C over tiles x splits workgroups.
template <class T, class C, bool RC, int EPI>
void launch_gemm(GemmArgs a, int splits, hipStream_t st) {
  fill_tiles<C>(a);
  // whole tiles, and every split's stage count even: no stage reads outside the operands
  const int per = a.red_per_split;
  const int last = a.red - (splits - 1) * per;
  const bool full = a.R % C::BR == 0 && a.C % C::BC == 0 && per % (2 * kBK) == 0 && last > 0 &&
                    last % (2 * kBK) == 0;
  if (full)
    hipLaunchKernelGGL((k_gemm<T, C, RC, RC, EPI, true>), dim3(a.tiles * splits), dim3(C::NT), 0, st, a);
  else
    hipLaunchKernelGGL((k_gemm<T, C, RC, RC, EPI, false>), dim3(a.tiles * splits), dim3(C::NT), 0, st, a);
}
template <class T, bool RC, int EPI>
void launch_gemm_auto(const GemmArgs& a, int splits, bool large, hipStream_t st) {
  if (large)
    launch_gemm<T, CfgL, RC, EPI>(a, splits, st);
  else
    launch_gemm<T, CfgS, RC, EPI>(a, splits, st);
}

template <class T>
el_status run_linear_fwd(const uint16_t* x, long ldx, int M, int K, const uint16_t* w, const float* bias,
                         int N, int relu, uint16_t* y, long ldy, hipStream_t st) {
  if (M == 0) return EL_OK;
  if (N == 1) {
    int L = 1;
    while (L < 64 && L * 8 < K) L *= 2;
    const int rows_per_block = 4 * (64 / L);
    const dim3 grid((M + rows_per_block - 1) / rows_per_block);
    switch (L) {
#define EL_GEMV_CASE(LL) \
  case LL: hipLaunchKernelGGL((k_gemv_fwd<T, LL>), grid, dim3(256), 0, st, x, ldx, M, K, w, bias, relu, y, ldy); break;
      EL_GEMV_CASE(1) EL_GEMV_CASE(2) EL_GEMV_CASE(4) EL_GEMV_CASE(8) EL_GEMV_CASE(16) EL_GEMV_CASE(32)
      EL_GEMV_CASE(64)
#undef EL_GEMV_CASE
    }
    return check_launch("el_linear_fwd");
  }
  GemmArgs a{};
  a.P = x; a.ldp = ldx; a.Q = w; a.ldq = K;
  a.R = M; a.C = N; a.red = K; a.red_per_split = (K + kBK - 1) / kBK * kBK;
  a.out = y; a.ldo = ldy; a.bias = bias; a.relu = relu;
  launch_gemm_auto<T, true, EPI_FWD>(a, 1, use_large(M, N), st);
  return check_launch("el_linear_fwd");
}

template <class T>
el_status run_linear_bwd(const uint16_t* x, long ldx, int M, int K, const uint16_t* w, int N,
                         const uint16_t* dz, long ldz, uint16_t* dx, long lddx, int mask,
                         float* dw, float* db, void* ws, hipStream_t st) {
  const WgradPlan pl = plan_wgrad(M, K, N);
  if (M == 0) {  // empty batch: zero gradients (a fill kernel, so the call stays capturable)
    const long n = static_cast<long>(N) * K;
    hipLaunchKernelGGL(k_fill_zero, dim3((n + 255) / 256), dim3(256), 0, st, dw, n);
    hipLaunchKernelGGL(k_fill_zero, dim3((N + 255) / 256), dim3(256), 0, st, db, static_cast<long>(N));
    return check_launch("el_linear_bwd");
  }
  if (N == 1) {
    if (dx) {
      const long nthr = static_cast<long>(M) * (K / 8);
      hipLaunchKernelGGL((k_gemv_dgrad<T>), dim3((nthr + 255) / 256), dim3(256), 0, st, dz, ldz, M, K, w,
                         mask ? x : nullptr, ldx, dx, lddx);
    }
    float* part = static_cast<float*>(ws);
    float* dbp = part + static_cast<size_t>(pl.splits) * K;
    hipLaunchKernelGGL((k_gemv_wgrad<T>), dim3(pl.splits), dim3(256), 0, st, x, ldx, M, K, dz, ldz, pl.per,
                       part, dbp);
    launch_split_sum(part, static_cast<long>(K), pl.splits, dw, dbp, 1, db, st);
    return check_launch("el_linear_bwd");
  }
  if (dx) {  // dx = dz w: with w transposed once into the workspace, both operands are
             // reduction-contiguous, as in the forward
    uint16_t* wt = static_cast<uint16_t*>(ws);
    const long nblk = static_cast<long>(N / 8) * (K / 8);
    hipLaunchKernelGGL(k_transpose16, dim3((nblk + 255) / 256), dim3(256), 0, st, w, wt, N, K);
    GemmArgs a{};
    a.P = dz; a.ldp = ldz; a.Q = wt; a.ldq = N;
    a.R = M; a.C = K; a.red = N; a.red_per_split = (N + kBK - 1) / kBK * kBK;
    a.out = dx; a.ldo = lddx; a.relu = mask; a.mask = x; a.ldm = ldx;
    launch_gemm_auto<T, true, EPI_DGRAD>(a, 1, use_large(M, K), st);
  }
  GemmArgs b{};
  b.P = dz; b.ldp = ldz; b.Q = x; b.ldq = ldx;
  b.R = N; b.C = K; b.red = M; b.red_per_split = pl.per;
  if (pl.splits == 1) {
    b.out = dw; b.ldo = K; b.split_stride = 0; b.dbp = db;
    launch_gemm_auto<T, false, EPI_WGRAD>(b, 1, pl.large, st);
  } else {
    float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + pl.wt_bytes);
    float* dbp = part + static_cast<size_t>(pl.splits) * N * K;
    b.out = part; b.ldo = K; b.split_stride = static_cast<long>(N) * K; b.dbp = dbp;
    launch_gemm_auto<T, false, EPI_WGRAD>(b, pl.splits, pl.large, st);
    launch_split_sum(part, static_cast<long>(N) * K, pl.splits, dw, dbp, N, db, st);
  }
  return check_launch("el_linear_bwd");
}

el_status check_linear(const char* fn, const void* x, int32_t ldx, int32_t M, int32_t K, const void* w,
                       int32_t N, el_dtype dtype) {
  if (dtype != EL_BF16 && dtype != EL_F16)
    return set_error(EL_ERR_UNSUPPORTED, std::string(fn) + ": dtype must be EL_BF16 or EL_F16");
  if (M < 0) return bad(fn, "M must be >= 0");
  if (K < 8 || K % 8 != 0) return set_error(EL_ERR_UNSUPPORTED, std::string(fn) + ": K must be a positive multiple of 8");
  if (N < 1) return bad(fn, "N must be >= 1");
  if (N != 1 && N % 8 != 0) return set_error(EL_ERR_UNSUPPORTED, std::string(fn) + ": N must be 1 or a multiple of 8");
  if (N == 1 && K > 2048) return set_error(EL_ERR_UNSUPPORTED, std::string(fn) + ": one-output layers take K <= 2048");
  if (ldx < K || ldx % 8 != 0) return bad(fn, "ldx must be >= K and a multiple of 8");
  if (!w || !al(w, 16)) return bad(fn, "w must be non-null and 16-byte aligned");
  if (M > 0 && (!x || !al(x, 16))) return bad(fn, "x must be non-null and 16-byte aligned");
  return EL_OK;
}

}  // namespace
}  // namespace el

using namespace el;

extern "C" {

EL_API el_status el_linear_fwd(const void* x, int32_t ldx, int32_t M, int32_t K, const void* w,
                               const float* bias, int32_t N, uint32_t act, void* y, int32_t ldy,
                               el_dtype dtype, hipStream_t stream) {
  const char* fn = "el_linear_fwd";
  const el_status s = check_linear(fn, x, ldx, M, K, w, N, dtype);
  if (s != EL_OK) return s;
  if (act != EL_ACT_NONE && act != EL_ACT_RELU) return bad(fn, "unknown activation");
  if (bias && !al(bias, 16)) return bad(fn, "bias must be 16-byte aligned");
  if (ldy < N || (N != 1 && ldy % 8 != 0)) return bad(fn, "ldy must be >= N (and a multiple of 8 when N > 1)");
  if (M > 0 && (!y || !al(y, N == 1 ? 2 : 16))) return bad(fn, "y must be non-null and aligned");
  const uint16_t* xs = static_cast<const uint16_t*>(x);
  const uint16_t* ws = static_cast<const uint16_t*>(w);
  uint16_t* ys = static_cast<uint16_t*>(y);
  const int relu = act == EL_ACT_RELU;
  return dtype == EL_BF16 ? run_linear_fwd<BF16T>(xs, ldx, M, K, ws, bias, N, relu, ys, ldy, stream)
                          : run_linear_fwd<F16T>(xs, ldx, M, K, ws, bias, N, relu, ys, ldy, stream);
}

EL_API size_t el_linear_bwd_workspace_bytes(int32_t M, int32_t K, int32_t N) {
  if (M < 0 || K < 1 || N < 1) return 0;
  return plan_wgrad(M, K, N).bytes;
}

EL_API el_status el_linear_bwd(const void* x, int32_t ldx, int32_t M, int32_t K, const void* w,
                               int32_t N, const void* dz, int32_t ldz, void* dx, int32_t lddx,
                               uint32_t flags, float* dw, float* db, el_dtype dtype,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "el_linear_bwd";
  const el_status s = check_linear(fn, x, ldx, M, K, w, N, dtype);
  if (s != EL_OK) return s;
  if (flags & ~static_cast<uint32_t>(EL_LINEAR_DX_RELU_MASK)) return bad(fn, "unknown flags");
  if (ldz < N || (N != 1 && ldz % 8 != 0)) return bad(fn, "ldz must be >= N (and a multiple of 8 when N > 1)");
  if (M > 0 && (!dz || !al(dz, N == 1 ? 2 : 16))) return bad(fn, "dz must be non-null and aligned");
  if (dx && (lddx < K || lddx % 8 != 0 || !al(dx, 16))) return bad(fn, "dx: lddx must be >= K, a multiple of 8, dx 16-byte aligned");
  if (!dx && (flags & EL_LINEAR_DX_RELU_MASK)) return bad(fn, "the ReLU mask flag needs dx");
  if (!dw || !db || !al(dw, 16) || !al(db, 4)) return bad(fn, "dw (16-byte aligned) and db must be non-null");
  const size_t need = plan_wgrad(M, K, N).bytes;
  if (need > 0 && (!workspace || !al(workspace, 256)))
    return set_error(EL_ERR_WORKSPACE, std::string(fn) + ": workspace must be non-null and 256-byte aligned");
  if (workspace_bytes < need) {
    char buf[160];
    std::snprintf(buf, sizeof buf, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes, need);
    return set_error(EL_ERR_WORKSPACE, buf);
  }
  const uint16_t* xs = static_cast<const uint16_t*>(x);
  const uint16_t* ws = static_cast<const uint16_t*>(w);
  const uint16_t* dzs = static_cast<const uint16_t*>(dz);
  uint16_t* dxs = static_cast<uint16_t*>(dx);
  const int mask = (flags & EL_LINEAR_DX_RELU_MASK) ? 1 : 0;
  return dtype == EL_BF16
             ? run_linear_bwd<BF16T>(xs, ldx, M, K, ws, N, dzs, ldz, dxs, lddx, mask, dw, db, workspace, stream)
             : run_linear_bwd<F16T>(xs, ldx, M, K, ws, N, dzs, ldz, dxs, lddx, mask, dw, db, workspace, stream);
}

EL_API el_status el_relu_bwd(const void* dy, const void* y, void* dz, int32_t M, int32_t N,
                             int32_t ld, el_dtype dtype, hipStream_t stream) {
  const char* fn = "el_relu_bwd";
  if (dtype != EL_BF16 && dtype != EL_F16)
    return set_error(EL_ERR_UNSUPPORTED, std::string(fn) + ": dtype must be EL_BF16 or EL_F16");
  if (M < 0 || N < 1) return bad(fn, "M must be >= 0 and N >= 1");
  if (N % 8 != 0 || ld < N || ld % 8 != 0)
    return set_error(EL_ERR_UNSUPPORTED, std::string(fn) + ": N and ld must be multiples of 8, ld >= N");
  if (M == 0) return EL_OK;
  if (!dy || !y || !dz || !al(dy, 16) || !al(y, 16) || !al(dz, 16)) return bad(fn, "null or misaligned pointer");
  const long n = static_cast<long>(M) * (N / 8);
  const dim3 grid(static_cast<unsigned>((n + 255) / 256));
  const uint16_t* a = static_cast<const uint16_t*>(dy);
  const uint16_t* b = static_cast<const uint16_t*>(y);
  uint16_t* c = static_cast<uint16_t*>(dz);
  if (dtype == EL_BF16)
    hipLaunchKernelGGL((k_relu_bwd<BF16T>), grid, dim3(256), 0, stream, a, b, c, M, N, static_cast<long>(ld));
  else
    hipLaunchKernelGGL((k_relu_bwd<F16T>), grid, dim3(256), 0, stream, a, b, c, M, N, static_cast<long>(ld));
  return check_launch(fn);
}

EL_API size_t el_bce_workspace_bytes(int32_t M) {
  if (M < 1) return 0;
  return static_cast<size_t>((static_cast<int64_t>(M) + kBceBlock - 1) / kBceBlock) * sizeof(double);
}

EL_API el_status el_bce_logits(const void* z, int32_t ldz, const float* labels, int32_t M,
                               el_dtype dtype, float* loss, void* dz, int32_t lddz, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "el_bce_logits";
  if (dtype != EL_BF16 && dtype != EL_F16)
    return set_error(EL_ERR_UNSUPPORTED, std::string(fn) + ": dtype must be EL_BF16 or EL_F16");
  if (M < 1) return bad(fn, "M must be >= 1");
  if (ldz < 1 || lddz < 1) return bad(fn, "ldz and lddz must be >= 1");
  if (!z || !labels || !loss || !dz || !al(z, 2) || !al(dz, 2) || !al(labels, 4) || !al(loss, 4))
    return bad(fn, "null or misaligned pointer");
  const size_t need = el_bce_workspace_bytes(M);
  if (!workspace || !al(workspace, 8) || workspace_bytes < need) {
    char buf[160];
    std::snprintf(buf, sizeof buf, "%s: workspace of %zu bytes (8-byte aligned), %zu needed", fn, workspace_bytes, need);
    return set_error(EL_ERR_WORKSPACE, buf);
  }
  const uint16_t* zs = static_cast<const uint16_t*>(z);
  uint16_t* dzs = static_cast<uint16_t*>(dz);
  double* part = static_cast<double*>(workspace);
  const int nb = (M + kBceBlock - 1) / kBceBlock;
  if (dtype == EL_BF16)
    hipLaunchKernelGGL((k_bce_grad<BF16T>), dim3(nb), dim3(kBceBlock), 0, stream, zs, static_cast<long>(ldz), labels,
                       M, dzs, static_cast<long>(lddz), part);
  else
    hipLaunchKernelGGL((k_bce_grad<F16T>), dim3(nb), dim3(kBceBlock), 0, stream, zs, static_cast<long>(ldz), labels,
                       M, dzs, static_cast<long>(lddz), part);
  hipLaunchKernelGGL(k_bce_sum, dim3(1), dim3(1024), 0, stream, part, nb, M, loss);
  return check_launch(fn);
}

EL_API el_status el_sgd_dense(float* master, void* copy, el_dtype copy_dtype, const float* grad,
                              int64_t n, float lr, hipStream_t stream) {
  const char* fn = "el_sgd_dense";
  if (n < 0) return bad(fn, "n must be >= 0");
  if (n == 0) return EL_OK;
  if (!master || !grad || !al(master, 4) || !al(grad, 4)) return bad(fn, "master and grad must be non-null");
  if (copy && copy_dtype != EL_BF16 && copy_dtype != EL_F16)
    return set_error(EL_ERR_UNSUPPORTED, std::string(fn) + ": copy dtype must be EL_BF16 or EL_F16");
  if (copy && !al(copy, 2)) return bad(fn, "copy must be 2-byte aligned");
  const dim3 grid(static_cast<unsigned>((n + 255) / 256));
  uint16_t* cs = static_cast<uint16_t*>(copy);
  if (!copy)
    hipLaunchKernelGGL(k_sgd_dense_f32, grid, dim3(256), 0, stream, master, grad, static_cast<long>(n), lr);
  else if (copy_dtype == EL_BF16)
    hipLaunchKernelGGL((k_sgd_dense<BF16T>), grid, dim3(256), 0, stream, master, cs, grad, static_cast<long>(n), lr);
  else
    hipLaunchKernelGGL((k_sgd_dense<F16T>), grid, dim3(256), 0, stream, master, cs, grad, static_cast<long>(n), lr);
  return check_launch(fn);
}

}  // extern "C"
