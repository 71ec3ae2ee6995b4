// abi.hip -- the extern "C" entry points of libembcore: host-side validation, then the
// launches.  Nothing is enqueued unless every argument checks out.
#include <cinttypes>
#include <cmath>
#include <cstdio>
#include <mutex>
#include <string>

#include "el_internal.hpp"

namespace el {

namespace {
thread_local std::string g_last_error;
}

el_status set_error(el_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

el_status check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(EL_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return EL_OK;
}

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

el_status bad(const char* fn, const char* what) {
  return set_error(EL_ERR_INVALID_ARG, std::string(fn) + ": " + what);
}

el_status check_tables(const el_tables* tab, const char* fn) {
  if (!tab) return bad(fn, "tables is null");
  if (tab->num_tables < 1) return bad(fn, "num_tables must be >= 1");
  if (tab->dim < 1) return bad(fn, "dim must be >= 1");
  if (!dtype_valid(tab->dtype)) return bad(fn, "unknown table dtype");
  if (tab->total_rows < 0 || tab->total_rows > 0xfffffffeLL)
    return bad(fn, "total_rows must be in [0, 2^32 - 1)");
  if (!tab->row_offset) return bad(fn, "row_offset is null");
  if (tab->total_rows > 0 && !tab->base) return bad(fn, "table base is null");
  if (!aligned(tab->base, 16)) return bad(fn, "table base must be 16-byte aligned");
  if ((tab->dim * dtype_size(tab->dtype)) % 16 != 0)
    return set_error(EL_ERR_UNSUPPORTED, std::string(fn) + ": dim * sizeof(dtype) must be a multiple of 16 bytes");
  if (!aligned(tab->row_offset, 8)) return bad(fn, "row_offset must be 8-byte aligned");
  if (tab->max_rows < 0 || tab->max_rows > tab->total_rows)
    return bad(fn, "max_rows must be in [0, total_rows]");
  return EL_OK;
}

el_status check_bags(const el_tables* tab, const el_bags* bags, const char* fn) {
  if (!bags) return bad(fn, "bags is null");
  if (bags->batch < 0) return bad(fn, "batch must be >= 0");
  const int64_t nbags = static_cast<int64_t>(tab->num_tables) * bags->batch;
  if (nbags + 1 >= (1LL << 31)) return bad(fn, "num_tables * batch + 1 must be < 2^31");
  if (bags->nnz < 0 || bags->nnz >= (1LL << 31)) return bad(fn, "nnz must be in [0, 2^31)");
  if (!bags->offsets) return bad(fn, "offsets is null");
  if (bags->nnz > 0 && !bags->indices) return bad(fn, "indices is null");
  if (!aligned(bags->offsets, 4) || !aligned(bags->indices, 4))
    return bad(fn, "indices / offsets must be 4-byte aligned");
  if (bags->nnz > 0 && tab->total_rows == 0) return bad(fn, "lookups into empty tables");
  return EL_OK;
}

el_status check_dense(const char* fn, const void* p, bool needed, const char* name) {
  if (needed && !p) return set_error(EL_ERR_INVALID_ARG, std::string(fn) + ": " + name + " is null");
  if (!aligned(p, 16)) return set_error(EL_ERR_INVALID_ARG, std::string(fn) + ": " + name + " must be 16-byte aligned");
  return EL_OK;
}

el_status check_interaction(const char* fn, int32_t B, int32_t F, int32_t D, int32_t out_stride,
                            el_dtype a, el_dtype b, el_dtype c) {
  if (B < 0) return bad(fn, "B must be >= 0");
  if (F < 1) return bad(fn, "F must be >= 1");
  if (D < 1) return bad(fn, "D must be >= 1");
  if (!dtype_valid(a) || !dtype_valid(b) || !dtype_valid(c)) return bad(fn, "unknown dtype");
  const int64_t V = static_cast<int64_t>(F) + 1;
  const int64_t P = V * (V - 1) / 2;
  if (static_cast<int64_t>(out_stride) < D + P) return bad(fn, "out_stride < D + (F+1)F/2");
  return EL_OK;
}

el_status check_cat(const char* fn, int32_t B, int32_t F, int32_t D, int32_t out_stride, el_dtype a,
                    el_dtype b) {
  if (B < 0) return bad(fn, "B must be >= 0");
  if (F < 1) return bad(fn, "F must be >= 1");
  if (D < 1) return bad(fn, "D must be >= 1");
  if (!dtype_valid(a) || !dtype_valid(b)) return bad(fn, "unknown dtype");
  const int64_t VD = (static_cast<int64_t>(F) + 1) * D;
  if (VD >= (1LL << 31)) return bad(fn, "(F+1) * D must be < 2^31");
  if (static_cast<int64_t>(out_stride) < VD) return bad(fn, "out_stride < (F+1) * D");
  return EL_OK;
}

// Scratch of emb_grad_reduce_update_noalloc (for callers that cannot allocate): one
// file-scope device array, of which every GPU the library runs on holds its own copy until
// the process ends.  In host code `scratch` only names the symbol; its device address on
// the current device comes from hipGetSymbolAddress, taken once per device and kept here.
constexpr size_t kNoallocScratchBytes = EL_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (resolved on the first call there).
el_status noalloc_scratch(const char* fn, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return set_error(EL_ERR_HIP, std::string(fn) + ": no usable current device");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return set_error(EL_ERR_HIP, std::string(fn) + ": hipGetSymbolAddress(scratch): " + hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return EL_OK;
}

#define EL_TRY(expr)                   \
  do {                                 \
    const el_status st_ = (expr);      \
    if (st_ != EL_OK) return st_;      \
  } while (0)

el_status check_grad_call(const char* fn, const el_tables* tab, const el_bags* bags, uint32_t flags,
                          void* workspace, size_t workspace_bytes) {
  EL_TRY(check_tables(tab, fn));
  EL_TRY(check_bags(tab, bags, fn));
  if (flags & ~static_cast<uint32_t>(EL_FLAG_HASH_INDICES)) return bad(fn, "unknown flags");
  const size_t need = plan_grad_workspace(*tab, bags->nnz, nullptr).bytes;
  if (need > 0) {
    if (!workspace) return set_error(EL_ERR_WORKSPACE, std::string(fn) + ": workspace is null");
    if (!aligned(workspace, 256)) return bad(fn, "workspace must be 256-byte aligned");
  }
  if (workspace_bytes < need) {
    char buf[160];
    std::snprintf(buf, sizeof buf, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes, need);
    return set_error(EL_ERR_WORKSPACE, buf);
  }
  return EL_OK;
}

el_status check_grad_input(const char* fn, const el_tables* tab, el_dtype grad_dtype) {
  if (!dtype_valid(grad_dtype)) return bad(fn, "unknown gradient dtype");
  if ((tab->dim * dtype_size(grad_dtype)) % 16 != 0)
    return set_error(EL_ERR_UNSUPPORTED, std::string(fn) + ": dim * sizeof(grad dtype) must be a multiple of 16 bytes");
  return EL_OK;
}

}  // namespace
}  // namespace el

using namespace el;

extern "C" {

el_status emb_bag_fwd(const el_tables* tab, const el_bags* bags, uint32_t flags, void* emb_out,
                      el_dtype out_dtype, hipStream_t stream) {
  const char* fn = "emb_bag_fwd";
  EL_TRY(check_tables(tab, fn));
  EL_TRY(check_bags(tab, bags, fn));
  if (flags & ~static_cast<uint32_t>(EL_FLAG_HASH_INDICES)) return bad(fn, "unknown flags");
  if (!dtype_valid(out_dtype)) return bad(fn, "unknown output dtype");
  const int64_t nbags = static_cast<int64_t>(tab->num_tables) * bags->batch;
  EL_TRY(check_dense(fn, emb_out, nbags > 0, "emb_out"));
  if (nbags == 0) return EL_OK;
  return launch_emb_bag_fwd(*tab, *bags, flags, emb_out, out_dtype, stream);
}

el_status dot_interact_fwd(const void* x0, const void* emb, el_dtype in_dtype, int32_t B, int32_t F,
                           int32_t D, void* out, el_dtype out_dtype, int32_t out_stride,
                           hipStream_t stream) {
  const char* fn = "dot_interact_fwd";
  EL_TRY(check_interaction(fn, B, F, D, out_stride, in_dtype, out_dtype, out_dtype));
  EL_TRY(check_dense(fn, x0, B > 0, "x0"));
  EL_TRY(check_dense(fn, emb, B > 0, "emb"));
  EL_TRY(check_dense(fn, out, B > 0, "out"));
  if (B == 0) return EL_OK;
  return launch_dot_fwd(x0, emb, in_dtype, B, F, D, out, out_dtype, out_stride, stream);
}

el_status dot_interact_bwd(const void* x0, const void* emb, el_dtype in_dtype, int32_t B, int32_t F,
                           int32_t D, const void* dout, el_dtype dout_dtype, int32_t out_stride,
                           void* dx0, void* demb, el_dtype grad_dtype, hipStream_t stream) {
  const char* fn = "dot_interact_bwd";
  EL_TRY(check_interaction(fn, B, F, D, out_stride, in_dtype, dout_dtype, grad_dtype));
  EL_TRY(check_dense(fn, x0, B > 0, "x0"));
  EL_TRY(check_dense(fn, emb, B > 0, "emb"));
  EL_TRY(check_dense(fn, dout, B > 0, "dout"));
  EL_TRY(check_dense(fn, dx0, B > 0, "dx0"));
  EL_TRY(check_dense(fn, demb, B > 0, "demb"));
  if (B == 0) return EL_OK;
  return launch_dot_bwd(x0, emb, in_dtype, B, F, D, dout, dout_dtype, out_stride, dx0, demb,
                        grad_dtype, stream);
}

el_status emb_dot_fwd(const el_tables* tab, const el_bags* bags, uint32_t flags, const void* x0,
                      el_dtype act_dtype, void* emb_out, void* out, int32_t out_stride,
                      hipStream_t stream) {
  const char* fn = "emb_dot_fwd";
  EL_TRY(check_tables(tab, fn));
  EL_TRY(check_bags(tab, bags, fn));
  if (flags & ~static_cast<uint32_t>(EL_FLAG_HASH_INDICES)) return bad(fn, "unknown flags");
  const int32_t B = bags->batch;
  EL_TRY(check_interaction(fn, B, tab->num_tables, tab->dim, out_stride, act_dtype, act_dtype, act_dtype));
  EL_TRY(check_dense(fn, x0, B > 0, "x0"));
  EL_TRY(check_dense(fn, emb_out, false, "emb_out"));
  EL_TRY(check_dense(fn, out, B > 0, "out"));
  if (B == 0) return EL_OK;
  return launch_emb_dot_fwd(*tab, *bags, flags, x0, act_dtype, emb_out, out, out_stride, stream);
}

el_status emb_dot_bwd(const el_tables* tab, const el_bags* bags, uint32_t flags, const void* x0,
                      el_dtype act_dtype, const void* dout, int32_t out_stride, void* dx0,
                      void* demb, el_dtype grad_dtype, hipStream_t stream) {
  const char* fn = "emb_dot_bwd";
  EL_TRY(check_tables(tab, fn));
  EL_TRY(check_bags(tab, bags, fn));
  if (flags & ~static_cast<uint32_t>(EL_FLAG_HASH_INDICES)) return bad(fn, "unknown flags");
  const int32_t B = bags->batch;
  EL_TRY(check_interaction(fn, B, tab->num_tables, tab->dim, out_stride, act_dtype, act_dtype, grad_dtype));
  EL_TRY(check_dense(fn, x0, B > 0, "x0"));
  EL_TRY(check_dense(fn, dout, B > 0, "dout"));
  EL_TRY(check_dense(fn, dx0, B > 0, "dx0"));
  EL_TRY(check_dense(fn, demb, B > 0, "demb"));
  if (B == 0) return EL_OK;
  return launch_emb_dot_bwd(*tab, *bags, flags, x0, act_dtype, dout, out_stride, dx0, demb,
                            grad_dtype, stream);
}

el_status cat_interact_fwd(const void* x0, const void* emb, el_dtype in_dtype, int32_t B, int32_t F,
                           int32_t D, void* out, el_dtype out_dtype, int32_t out_stride,
                           hipStream_t stream) {
  const char* fn = "cat_interact_fwd";
  EL_TRY(check_cat(fn, B, F, D, out_stride, in_dtype, out_dtype));
  EL_TRY(check_dense(fn, x0, B > 0, "x0"));
  EL_TRY(check_dense(fn, emb, B > 0, "emb"));
  EL_TRY(check_dense(fn, out, B > 0, "out"));
  if (B == 0) return EL_OK;
  return launch_cat_fwd(x0, emb, in_dtype, B, F, D, out, out_dtype, out_stride, stream);
}

el_status cat_interact_bwd(const void* dout, el_dtype dout_dtype, int32_t B, int32_t F, int32_t D,
                           int32_t out_stride, void* dx0, void* demb, el_dtype grad_dtype,
                           hipStream_t stream) {
  const char* fn = "cat_interact_bwd";
  EL_TRY(check_cat(fn, B, F, D, out_stride, dout_dtype, grad_dtype));
  EL_TRY(check_dense(fn, dout, B > 0, "dout"));
  EL_TRY(check_dense(fn, dx0, B > 0, "dx0"));
  EL_TRY(check_dense(fn, demb, B > 0, "demb"));
  if (B == 0) return EL_OK;
  return launch_cat_bwd(dout, dout_dtype, B, F, D, out_stride, dx0, demb, grad_dtype, stream);
}

el_status emb_cat_fwd(const el_tables* tab, const el_bags* bags, uint32_t flags, const void* x0,
                      el_dtype act_dtype, void* out, int32_t out_stride, hipStream_t stream) {
  const char* fn = "emb_cat_fwd";
  EL_TRY(check_tables(tab, fn));
  EL_TRY(check_bags(tab, bags, fn));
  if (flags & ~static_cast<uint32_t>(EL_FLAG_HASH_INDICES)) return bad(fn, "unknown flags");
  const int32_t B = bags->batch;
  EL_TRY(check_cat(fn, B, tab->num_tables, tab->dim, out_stride, act_dtype, act_dtype));
  EL_TRY(check_dense(fn, x0, B > 0, "x0"));
  EL_TRY(check_dense(fn, out, B > 0, "out"));
  if (B == 0) return EL_OK;
  return launch_emb_cat_fwd(*tab, *bags, flags, x0, act_dtype, out, out_stride, stream);
}

size_t emb_grad_workspace_bytes(const el_tables* tab, const el_bags* bags) {
  if (check_tables(tab, "emb_grad_workspace_bytes") != EL_OK) return 0;
  if (check_bags(tab, bags, "emb_grad_workspace_bytes") != EL_OK) return 0;
  return plan_grad_workspace(*tab, bags->nnz, nullptr).bytes;
}


el_status emb_grad_reduce_update(const el_tables* tab, const el_bags* bags, uint32_t flags,
                                 const void* demb, el_dtype grad_dtype, float lr, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "emb_grad_reduce_update";
  EL_TRY(check_grad_call(fn, tab, bags, flags, workspace, workspace_bytes));
  EL_TRY(check_grad_input(fn, tab, grad_dtype));
  if (bags->batch == 0 || bags->nnz == 0) return EL_OK;
  EL_TRY(check_dense(fn, demb, true, "demb"));
  GradWorkspace ws = plan_grad_workspace(*tab, bags->nnz, workspace);
  uint32_t *keys = nullptr, *vals = nullptr;
  EL_TRY(launch_grad_sort_core(*tab, *bags, flags, ws, &keys, &vals, stream));
  return launch_reduce_update(*tab, *bags, ws, keys, vals, demb, grad_dtype, lr, stream);
}

el_status emb_grad_reduce_update_noalloc(const el_tables* tab, const el_bags* bags, uint32_t flags,
                                         const void* demb, el_dtype grad_dtype, float lr,
                                         hipStream_t stream) {
  const char* fn = "emb_grad_reduce_update_noalloc";
  EL_TRY(check_tables(tab, fn));
  EL_TRY(check_bags(tab, bags, fn));
  if (flags & ~static_cast<uint32_t>(EL_FLAG_HASH_INDICES)) return bad(fn, "unknown flags");
  EL_TRY(check_grad_input(fn, tab, grad_dtype));
  if (bags->batch == 0 || bags->nnz == 0) return EL_OK;
  EL_TRY(check_dense(fn, demb, true, "demb"));
  const size_t need = plan_grad_workspace(*tab, bags->nnz, nullptr).bytes;
  if (need > kNoallocScratchBytes) {
    char buf[200];
    std::snprintf(buf, sizeof buf, "%s: %zu bytes of scratch needed, the library's static scratch holds %zu",
                  fn, need, kNoallocScratchBytes);
    return set_error(EL_ERR_WORKSPACE, buf);
  }
  void* scratch_ptr = nullptr;
  EL_TRY(noalloc_scratch(fn, &scratch_ptr));
  GradWorkspace ws = plan_grad_workspace(*tab, bags->nnz, scratch_ptr);
  uint32_t *keys = nullptr, *vals = nullptr;
  EL_TRY(launch_grad_sort_core(*tab, *bags, flags, ws, &keys, &vals, stream));
  return launch_reduce_update(*tab, *bags, ws, keys, vals, demb, grad_dtype, lr, stream);
}

el_status emb_grad_prepare(const el_tables* tab, const el_bags* bags, uint32_t flags, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "emb_grad_prepare";
  EL_TRY(check_grad_call(fn, tab, bags, flags, workspace, workspace_bytes));
  if (bags->batch == 0 || bags->nnz == 0) return EL_OK;
  GradWorkspace ws = plan_grad_workspace(*tab, bags->nnz, workspace);
  uint32_t *keys = nullptr, *vals = nullptr;
  return launch_grad_sort_core(*tab, *bags, flags, ws, &keys, &vals, stream);
}

el_status emb_grad_apply(const el_tables* tab, const el_bags* bags, uint32_t flags, const void* demb,
                         el_dtype grad_dtype, float lr, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  const char* fn = "emb_grad_apply";
  EL_TRY(check_grad_call(fn, tab, bags, flags, workspace, workspace_bytes));
  EL_TRY(check_grad_input(fn, tab, grad_dtype));
  if (bags->batch == 0 || bags->nnz == 0) return EL_OK;
  EL_TRY(check_dense(fn, demb, true, "demb"));
  GradWorkspace ws = plan_grad_workspace(*tab, bags->nnz, workspace);
  uint32_t *keys = nullptr, *vals = nullptr;
  sorted_buffers(ws, &keys, &vals);
  return launch_reduce_update(*tab, *bags, ws, keys, vals, demb, grad_dtype, lr, stream);
}

el_status emb_grad_sort(const el_tables* tab, const el_bags* bags, uint32_t flags, void* workspace,
                        size_t workspace_bytes, uint32_t* sorted_rows, uint32_t* bag_ids,
                        uint32_t* unique_rows, uint32_t* seg_offsets, uint32_t* num_unique,
                        hipStream_t stream) {
  const char* fn = "emb_grad_sort";
  EL_TRY(check_grad_call(fn, tab, bags, flags, workspace, workspace_bytes));
  if (!seg_offsets || !num_unique) return bad(fn, "seg_offsets / num_unique is null");
  const bool any = bags->batch > 0 && bags->nnz > 0;
  if (any && (!sorted_rows || !bag_ids || !unique_rows)) return bad(fn, "output array is null");
  GradWorkspace ws = plan_grad_workspace(*tab, any ? bags->nnz : 0, workspace);
  if (!any) return launch_segments(ws, nullptr, unique_rows, seg_offsets, num_unique, stream);
  uint32_t *keys = nullptr, *vals = nullptr;
  EL_TRY(launch_grad_sort_core(*tab, *bags, flags, ws, &keys, &vals, stream));
  const size_t bytes = sizeof(uint32_t) * static_cast<size_t>(ws.n);
  if (hipMemcpyAsync(sorted_rows, keys, bytes, hipMemcpyDeviceToDevice, stream) != hipSuccess ||
      hipMemcpyAsync(bag_ids, vals, bytes, hipMemcpyDeviceToDevice, stream) != hipSuccess)
    return check_launch("emb_grad_sort copy");
  return launch_segments(ws, keys, unique_rows, seg_offsets, num_unique, stream);
}

el_status el_validate_bags(const el_tables* tab, const el_bags* bags, uint32_t flags,
                           int64_t* bad_count, hipStream_t stream) {
  const char* fn = "el_validate_bags";
  EL_TRY(check_tables(tab, fn));
  if (!bags) return bad(fn, "bags is null");
  if (bags->batch < 0) return bad(fn, "batch must be >= 0");
  if (static_cast<int64_t>(tab->num_tables) * bags->batch + 1 >= (1LL << 31))
    return bad(fn, "num_tables * batch + 1 must be < 2^31");
  if (bags->nnz < 0 || bags->nnz >= (1LL << 31)) return bad(fn, "nnz must be in [0, 2^31)");
  if (!bags->offsets) return bad(fn, "offsets is null");
  if (bags->nnz > 0 && !bags->indices) return bad(fn, "indices is null");
  if (!bad_count || !aligned(bad_count, 8)) return bad(fn, "bad_count must be a non-null 8-byte aligned pointer");
  return launch_validate(*tab, *bags, flags, bad_count, stream);
}

el_status el_hbm_calib(int32_t mode, const void* src, void* dst, size_t bytes, const int32_t* idx,
                       int64_t nrows, int32_t row_bytes, hipStream_t stream) {
  const char* fn = "el_hbm_calib";
  const int32_t policy = mode & ~EL_CALIB_MODE_MASK;
  const int32_t full = mode;
  mode &= EL_CALIB_MODE_MASK;
  if (mode > EL_CALIB_GATHER_READ || (policy & ~(EL_CALIB_NT_LOADS | EL_CALIB_NT_STORES)) != 0)
    return bad(fn, "unknown mode");
  EL_TRY(check_dense(fn, dst, true, "dst"));
  if (mode == EL_CALIB_GATHER || mode == EL_CALIB_GATHER_READ) {
    EL_TRY(check_dense(fn, src, true, "src"));
    if (!idx || !aligned(idx, 4)) return bad(fn, "idx must be a non-null 4-byte aligned pointer");
    if (nrows < 0) return bad(fn, "nrows must be >= 0");
    if (row_bytes < 16 || row_bytes > 1024 || row_bytes % 16 != 0)
      return bad(fn, "row_bytes must be a multiple of 16 in [16, 1024]");
    if (mode == EL_CALIB_GATHER && (bytes % 16 != 0 || bytes > static_cast<size_t>(row_bytes)))
      return bad(fn, "bytes written per gathered row must be a multiple of 16, at most row_bytes");
    if (nrows == 0) return EL_OK;
  } else {
    if (mode != EL_CALIB_WRITE) EL_TRY(check_dense(fn, src, true, "src"));
    if (bytes % 64 != 0) return bad(fn, "bytes must be a multiple of 64");
    if (bytes == 0) return EL_OK;
  }
  return launch_hbm_calib(full, src, dst, bytes, idx, nrows, row_bytes, stream);
}

const char* el_last_error(void) { return g_last_error.c_str(); }

int el_version(void) { return 200; }

}  // extern "C"

// ---------------------------------------------------------------------------------------
// el_validate_bags kernels: a grid of workgroups over the bags, each thread counting the
// defects of its bags; workgroup subtotals are added to the count with one 64-bit integer
// atomic each (an exact integer sum, the same for any order).  The count is cleared by a
// one-thread kernel first (a kernel rather than a memset, so that the call can be captured
// in a HIP graph).
// ---------------------------------------------------------------------------------------
namespace el {
namespace {

__global__ void k_validate_clear(int64_t* __restrict__ bad_count) {
  if (threadIdx.x == 0) bad_count[0] = 0;
}

__global__ __launch_bounds__(256) void k_validate(const int64_t* __restrict__ row_off,
                                                  const int32_t* __restrict__ idx,
                                                  const int32_t* __restrict__ off, int32_t F,
                                                  int32_t B, int64_t nnz, uint32_t hash,
                                                  int64_t max_rows, int64_t* __restrict__ bad_count) {
  __shared__ int64_t part[4];
  const int64_t nbags = static_cast<int64_t>(F) * B;
  int64_t bad = 0;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    if (off[0] != 0) ++bad;
    if (off[nbags] != nnz) ++bad;
  }
  if (blockIdx.x == 0 && max_rows > 0)  // tables larger than the declared largest
    for (int t = threadIdx.x; t < F; t += 256)
      if (row_off[t + 1] - row_off[t] > max_rows) ++bad;
  for (int64_t g = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; g < nbags;
       g += static_cast<int64_t>(gridDim.x) * 256) {
    const int32_t s = off[g], e = off[g + 1];
    if (e < s) ++bad;
    if (!hash) {
      const int t = static_cast<int>(g / B);
      const int64_t n = row_off[t + 1] - row_off[t];
      const int64_t lo = s < 0 ? 0 : s;
      const int64_t hi = e > nnz ? nnz : e;
      for (int64_t k = lo; k < hi; ++k) {
        const int32_t r = idx[k];
        if (r < 0 || r >= n) ++bad;
      }
    }
  }
  // wavefront sums, then the workgroup's four wave sums, added to the count
  for (int o = 32; o > 0; o >>= 1) bad += __shfl_down(bad, o);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = bad;
  __syncthreads();
  if (threadIdx.x == 0) {
    const int64_t tot = part[0] + part[1] + part[2] + part[3];
    if (tot) atomicAdd(reinterpret_cast<unsigned long long*>(bad_count), static_cast<unsigned long long>(tot));
  }
}

}  // namespace

el_status launch_validate(const el_tables& tab, const el_bags& bags, uint32_t flags,
                          int64_t* bad_count, hipStream_t stream) {
  hipLaunchKernelGGL(k_validate_clear, dim3(1), dim3(64), 0, stream, bad_count);
  el_status st = check_launch("el_validate_bags");
  if (st != EL_OK) return st;
  const int64_t nbags = static_cast<int64_t>(tab.num_tables) * bags.batch;
  int64_t blocks = (nbags + 255) / 256;
  blocks = blocks < 1 ? 1 : (blocks > 4096 ? 4096 : blocks);
  hipLaunchKernelGGL(k_validate, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, tab.row_offset,
                     bags.indices, bags.offsets, tab.num_tables, bags.batch, bags.nnz,
                     (flags & EL_FLAG_HASH_INDICES) ? 1u : 0u, tab.max_rows, bad_count);
  return check_launch("el_validate_bags");
}

}  // namespace el
