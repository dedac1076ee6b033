// Calls every entry point of the HIP library's C ABI with invalid arguments
// (null, misaligned, out-of-range sizes, zero queries) under AddressSanitizer
// / UBSan in the host code.  Every such call returns its status before any
// HIP call, so no GPU is needed.  Prints one status per call.  Test
// infrastructure only.
#include <cstdint>
#include <cstdio>

#include "sparse_attn.h"

int main() {
    void *A = reinterpret_cast<void *>(0x10000), *A2 = reinterpret_cast<void *>(0x20000);
    void *MIS = reinterpret_cast<void *>(0x10002);
    const int32_t *I = reinterpret_cast<const int32_t *>(0x10000);
    const float *FR = reinterpret_cast<const float *>(0x10000);
    sa_dims d{2, 3, 64, 512, 100, 40};
    sa_dims dz{0, 3, 64, 512, 100, 40};
    sa_dims dbadD{2, 3, 64, 100, 100, 40};
    sa_dims dbigK{2, 3, 64, 512, 100, 4096};
    sa_dims dneg{2, -1, 64, 512, 100, 40};
    int n = 0;
    auto show = [&](const char *what, long long v) { std::printf("%02d %s %lld\n", n++, what, v); };
    show("fwd null dims", sparse_attn_fwd(A, A, nullptr, I, 0.1f, A2, nullptr, nullptr, 0, nullptr));
    show("fwd bad D", sparse_attn_fwd(A, A, nullptr, I, 0.1f, A2, &dbadD, nullptr, 0, nullptr));
    show("fwd big K", sparse_attn_fwd(A, A, nullptr, I, 0.1f, A2, &dbigK, nullptr, 0, nullptr));
    show("fwd neg T", sparse_attn_fwd(A, A, nullptr, I, 0.1f, A2, &dneg, nullptr, 0, nullptr));
    show("fwd null q", sparse_attn_fwd(nullptr, A, nullptr, I, 0.1f, A2, &d, nullptr, 0, nullptr));
    show("fwd misaligned out", sparse_attn_fwd(A, A, nullptr, I, 0.1f, MIS, &d, nullptr, 0, nullptr));
    show("fwd zero queries", sparse_attn_fwd(nullptr, nullptr, nullptr, nullptr, 0.1f, nullptr, &dz, nullptr, 0, nullptr));
    show("splits -1", sparse_attn_fwd_splits(A, A, nullptr, I, 0.1f, A2, &d, -1, nullptr, 0, nullptr));
    show("splits 2 no ws", sparse_attn_fwd_splits(A, A, nullptr, I, 0.1f, A2, &d, 2, nullptr, 0, nullptr));
    show("splits 2 small ws", sparse_attn_fwd_splits(A, A, nullptr, I, 0.1f, A2, &d, 2, A, 16, nullptr));
    show("ws bytes S=4", (long long)sparse_attn_workspace_bytes_splits(&d, 4));
    show("ws bytes bad", (long long)sparse_attn_workspace_bytes_splits(&dbadD, 4));
    show("ws bytes planned bad", (long long)sparse_attn_workspace_bytes(&dbadD));
    show("rope bad rd", sparse_attn_fwd_rope(A, A, nullptr, I, 0.1f, FR, 7, A2, &d, 1, nullptr, 0, nullptr));
    show("2src bad W", sparse_attn_fwd_2src(A, A, 10, A, 10, 200, nullptr, I, 0.1f, A2, &d, 1, nullptr, 0, nullptr));
    show("fp4 record bytes", sparse_attn_fp4_record_bytes(512));
    show("fp4 null dims", sparse_attn_fwd_2src_fp4(A, A, 10, A, 100, 10, nullptr, I, 0.1f, A2, nullptr, 1, nullptr, 0, nullptr));
    show("partial S=1", sparse_attn_fwd_partial(A, A, I, 0.1f, &d, 1, A, 1 << 30, nullptr));
    show("combine no ws", sparse_attn_fwd_combine(nullptr, A, &d, 2, nullptr, 1 << 30, nullptr));
    show("noalloc S=65", sparse_attn_fwd_noalloc(A, A, nullptr, I, 0.1f, A2, &d, 65, nullptr));
    sa_dims dhuge{512, 1, 64, 512, 1024, 640};
    show("noalloc too big", sparse_attn_fwd_noalloc(A, A, nullptr, I, 0.1f, A2, &dhuge, 64, nullptr));
    show("check null", sparse_attn_check_idxs(nullptr, &d, reinterpret_cast<int32_t *>(A), nullptr));
    show("topk bad stride", sparse_attn_topk(reinterpret_cast<const float *>(A), nullptr, 4, 100, 10, 0,
                                             reinterpret_cast<int32_t *>(A), 5, nullptr));
    show("plan kernel bad", sparse_attn_plan_kernel(&dbadD, 0) == nullptr ? 1 : 0);
    std::printf("status 99: %s\n", sparse_attn_status_str(99));
    return 0;
}
