// The C ABI's host-side checks under AddressSanitizer and UndefinedBehaviorSanitizer (test
// infrastructure; CPU only, no GPU needed).
//
// The library's sources are built with the sanitizers on their host code only and linked
// into this program, which calls every entry point with arguments its checks must refuse
// (null, misaligned, negative, oversize and inconsistent shapes, unknown dtypes, flags and
// modes) and the pure host size queries over ordinary and extreme sizes, where an integer
// overflow would be undefined behaviour.  Nothing is enqueued on a GPU: every call stops
// at its checks.  Prints "ok" and exits 0 when every call returned what the header promises.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "embcore.h"

static int failures = 0;

#define EXPECT(cond)                                               \
  do {                                                             \
    if (!(cond)) {                                                 \
      std::printf("FAIL line %d: %s\n", __LINE__, #cond);          \
      ++failures;                                                  \
    }                                                              \
  } while (0)

// An error status, with a message that names the call.
#define REFUSED(call, name)                                                      \
  do {                                                                           \
    const el_status st_ = (call);                                                \
    EXPECT(st_ == EL_ERR_INVALID_ARG || st_ == EL_ERR_UNSUPPORTED || st_ == EL_ERR_WORKSPACE); \
    EXPECT(std::strstr(el_last_error(), name) != nullptr);                       \
  } while (0)

static void* addr(uintptr_t a) { return reinterpret_cast<void*>(a); }

int main() {
  const uintptr_t A = 0x7F0000000000ull;  // aligned stand-in device addresses, never used
  const int64_t* ro = static_cast<const int64_t*>(addr(A + 0x1000));
  const int32_t* ip = static_cast<const int32_t*>(addr(A + 0x2000));
  const int32_t* op = static_cast<const int32_t*>(addr(A + 0x3000));
  el_tables T{addr(A), ro, 26LL * 100000, 26, 128, EL_F32, 0};
  el_bags Bg{ip, op, 65536, 26LL * 65536};

  // gather and fused calls
  REFUSED(emb_bag_fwd(nullptr, &Bg, 0, addr(A), EL_BF16, nullptr), "emb_bag_fwd");
  el_tables t0 = T; t0.num_tables = 0;
  REFUSED(emb_bag_fwd(&t0, &Bg, 0, addr(A), EL_BF16, nullptr), "emb_bag_fwd");
  el_tables t3 = T; t3.dim = 3;
  REFUSED(emb_bag_fwd(&t3, &Bg, 0, addr(A), EL_BF16, nullptr), "emb_bag_fwd");
  el_tables tm = T; tm.base = addr(A + 8);
  REFUSED(emb_bag_fwd(&tm, &Bg, 0, addr(A), EL_BF16, nullptr), "emb_bag_fwd");
  el_bags bbig = Bg; bbig.nnz = int64_t(1) << 31;
  REFUSED(emb_bag_fwd(&T, &bbig, 0, addr(A), EL_BF16, nullptr), "emb_bag_fwd");
  el_bags bneg = Bg; bneg.batch = -1;
  REFUSED(emb_bag_fwd(&T, &bneg, 0, addr(A), EL_BF16, nullptr), "emb_bag_fwd");
  REFUSED(emb_bag_fwd(&T, &Bg, 2, addr(A), EL_BF16, nullptr), "emb_bag_fwd");
  REFUSED(emb_bag_fwd(&T, &Bg, 0, addr(A + 4), EL_BF16, nullptr), "emb_bag_fwd");
  REFUSED(emb_bag_fwd(&T, &Bg, 0, addr(A), static_cast<el_dtype>(7), nullptr), "emb_bag_fwd");
  el_tables tbad = T; tbad.dtype = static_cast<el_dtype>(9);
  REFUSED(emb_bag_fwd(&tbad, &Bg, 0, addr(A), EL_BF16, nullptr), "emb_bag_fwd");
  el_bags bnull = Bg; bnull.offsets = nullptr;
  REFUSED(emb_bag_fwd(&T, &bnull, 0, addr(A), EL_BF16, nullptr), "emb_bag_fwd");
  el_bags bhuge = Bg; bhuge.batch = 0x7fffffff;  // F * B beyond 32 bits
  REFUSED(emb_bag_fwd(&T, &bhuge, 0, addr(A), EL_BF16, nullptr), "emb_bag_fwd");
  REFUSED(emb_dot_fwd(&T, &Bg, 0, addr(A), EL_BF16, addr(A), addr(A), 478, nullptr), "emb_dot_fwd");
  REFUSED(emb_dot_fwd(&T, &Bg, 0, nullptr, EL_BF16, addr(A), addr(A), 480, nullptr), "emb_dot_fwd");
  REFUSED(emb_dot_fwd(&T, &Bg, 0, addr(A), EL_F32, nullptr, addr(A), 480, nullptr), "emb_dot_fwd");
  REFUSED(emb_cat_fwd(&T, &Bg, 0, addr(A), EL_BF16, addr(A), 27 * 128 - 8, nullptr), "emb_cat_fwd");
  REFUSED(emb_dot_bwd(&T, &Bg, 0, addr(A), EL_BF16, addr(A), 478, addr(A), addr(A), EL_BF16, nullptr),
          "emb_dot_bwd");

  // interaction calls
  REFUSED(dot_interact_fwd(addr(A), addr(A), EL_BF16, 65536, 26, 128, addr(A), EL_BF16, 478, nullptr),
          "dot_interact_fwd");
  REFUSED(dot_interact_fwd(addr(A), addr(A), EL_BF16, -1, 26, 128, addr(A), EL_BF16, 480, nullptr),
          "dot_interact_fwd");
  REFUSED(dot_interact_fwd(addr(A), addr(A), EL_BF16, 65536, 0x7fffffff, 128, addr(A), EL_BF16, 480, nullptr),
          "dot_interact_fwd");
  REFUSED(dot_interact_bwd(addr(A), addr(A), EL_BF16, 65536, 26, 128, addr(A), EL_BF16, 480, nullptr, addr(A),
                           EL_BF16, nullptr), "dot_interact_bwd");
  REFUSED(dot_interact_bwd(addr(A), addr(A + 2), EL_BF16, 65536, 26, 128, addr(A), EL_BF16, 480, addr(A),
                           addr(A), EL_BF16, nullptr), "dot_interact_bwd");
  REFUSED(cat_interact_fwd(addr(A), addr(A), EL_BF16, 65536, 26, 128, addr(A), EL_BF16, 100, nullptr),
          "cat_interact_fwd");
  REFUSED(cat_interact_bwd(addr(A), EL_BF16, 65536, 26, 128, 100, addr(A), addr(A), EL_BF16, nullptr),
          "cat_interact_bwd");

  // the gradient path: size queries (pure host arithmetic) and refusals
  const size_t ws = emb_grad_workspace_bytes(&T, &Bg);
  EXPECT(ws >= size_t(6) * 4 * 26 * 65536);
  el_bags bempty = Bg; bempty.batch = 0; bempty.nnz = 0;
  EXPECT(emb_grad_workspace_bytes(&T, &bempty) == 0);
  EXPECT(emb_grad_workspace_bytes(nullptr, &Bg) == 0);
  el_tables tmax = T; tmax.max_rows = T.total_rows + 1;
  EXPECT(emb_grad_workspace_bytes(&tmax, &Bg) == 0);
  el_tables tneg = T; tneg.max_rows = -1;
  EXPECT(emb_grad_workspace_bytes(&tneg, &Bg) == 0);
  el_bags bmax = Bg; bmax.batch = 0x7fffffff / 26; bmax.nnz = (int64_t(1) << 31) - 1;
  (void)emb_grad_workspace_bytes(&T, &bmax);  // largest accepted lookup count: no overflow
  el_tables thuge = T; thuge.total_rows = (int64_t(1) << 32) - 1;
  (void)emb_grad_workspace_bytes(&thuge, &Bg);
  REFUSED(emb_grad_reduce_update(&T, &Bg, 0, addr(A), EL_BF16, 0.01f, addr(A), ws - 1, nullptr),
          "emb_grad_reduce_update");
  REFUSED(emb_grad_reduce_update(&T, &Bg, 0, nullptr, EL_BF16, 0.01f, addr(A), ws, nullptr),
          "emb_grad_reduce_update");
  REFUSED(emb_grad_prepare(&T, &Bg, 0, addr(A), ws - 1, nullptr), "emb_grad_prepare");
  REFUSED(emb_grad_apply(&T, &Bg, 0, addr(A), EL_BF16, 0.01f, addr(A), ws - 1, nullptr), "emb_grad_apply");
  REFUSED(emb_grad_sort(&T, &Bg, 0, addr(A), ws, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr),
          "emb_grad_sort");
  REFUSED(emb_grad_reduce_update_noalloc(&T, &Bg, 4, addr(A), EL_BF16, 0.01f, nullptr),
          "emb_grad_reduce_update_noalloc");
  REFUSED(el_validate_bags(&T, &Bg, 0, nullptr, nullptr), "el_validate_bags");

  // dense layers, loss and SGD
  const int32_t big = 0x7fffffff;
  EXPECT(el_linear_bwd_workspace_bytes(65536, 1024, 1024) > 0);
  (void)el_linear_bwd_workspace_bytes(big, 8, 8);
  (void)el_linear_bwd_workspace_bytes(big, 2048, 1);
  (void)el_linear_bwd_workspace_bytes(65536, big - 7, 8);
  (void)el_linear_bwd_workspace_bytes(0, 8, 8);
  (void)el_linear_bwd_workspace_bytes(-1, 8, 8);
  EXPECT(el_bce_workspace_bytes(65536) > 0);
  (void)el_bce_workspace_bytes(big);
  (void)el_bce_workspace_bytes(0);
  (void)el_bce_workspace_bytes(-5);
  REFUSED(el_linear_fwd(addr(A), 7, 64, 7, addr(A), nullptr, 8, 0, addr(A), 8, EL_BF16, nullptr), "el_linear_fwd");
  REFUSED(el_linear_fwd(addr(A), 16, 64, 16, addr(A), nullptr, 8, 0, addr(A), 8, EL_F32, nullptr), "el_linear_fwd");
  REFUSED(el_linear_bwd(addr(A), 16, 64, 16, addr(A), 8, addr(A), 8, addr(A), 16, 0, nullptr,
                        static_cast<float*>(addr(A)), EL_BF16, addr(A), 1 << 20, nullptr), "el_linear_bwd");
  REFUSED(el_relu_bwd(addr(A), addr(A), addr(A), 64, 16, 8, EL_BF16, nullptr), "el_relu_bwd");
  REFUSED(el_bce_logits(addr(A), 1, nullptr, 64, EL_BF16, static_cast<float*>(addr(A)), addr(A), 1, addr(A),
                        1 << 20, nullptr), "el_bce_logits");
  REFUSED(el_sgd_dense(nullptr, nullptr, EL_BF16, static_cast<const float*>(addr(A)), 16, 0.1f, nullptr),
          "el_sgd_dense");
  REFUSED(el_sgd_dense(static_cast<float*>(addr(A)), nullptr, EL_BF16, static_cast<const float*>(addr(A)), -1,
                       0.1f, nullptr), "el_sgd_dense");
  REFUSED(el_hbm_calib(999, addr(A), addr(A), 1 << 20, nullptr, 0, 0, nullptr), "el_hbm_calib");
  REFUSED(el_hbm_calib(1 | 64, addr(A), addr(A), 1 << 20, nullptr, 0, 0, nullptr), "el_hbm_calib");

  EXPECT(el_version() > 0);
  EXPECT(el_last_error() != nullptr);
  if (failures) {
    std::printf("%d failures\n", failures);
    return 1;
  }
  std::printf("ok\n");
  return 0;
}
