// lsa_sparse_attend without a caller workspace: the split-key partial
// results and arrival words live in a fixed device array of this library.
//
// lsa_sparse_attend needs a workspace only when few (query, KV head) units
// are spread over several key-list splits (decode), and then at most about
// 1024 units x splits, i.e. 1024 x G x (d + 2) x 4 + units x 8 bytes.  The
// array below holds kNoAllocScratchBytes; a call that would need more is
// rejected.  Every call on a device shares that device's copy of the array:
// calls that overlap in time on one device race (run them on one stream, or
// order them).  Nothing in it needs clearing: the partials are written
// before they are read, and an arrival word left by an earlier call carries
// that call's tag, so the next call's first arrival claims it afresh.

#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/lsa.h"
#include "lsa_launch.hpp"

namespace {

constexpr size_t kNoAllocScratchBytes = (size_t)4 << 20;   // 4 MiB per device
constexpr int kMaxDevices = 64;

// The library's own workspace: one copy per device, alive until the process ends.  In host code this
// name is only a handle for hipGetSymbolAddress; kernels receive the device address looked up below.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of this device's copy of the array, looked up once per device (with the device
// current); nullptr on failure, with the error recorded.
void* scratch_for_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        lsa::set_error(LSA_ERR_HIP, "lsa_sparse_attend_noalloc: no current HIP device");
        return nullptr;
    }
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || ptr == nullptr) {
            lsa::set_error(LSA_ERR_HIP, "lsa_sparse_attend_noalloc: hipGetSymbolAddress of the scratch array failed");
            return nullptr;
        }
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" lsa_status lsa_sparse_attend_noalloc(const lsa_layout* layout, const lsa_select_cfg* cfg, const void* Q,
                                                const void* K, const void* V, int64_t t_cap, int64_t T,
                                                const int64_t* q_pos, int64_t batch, int64_t n_q,
                                                const int32_t* lr_idx, const int32_t* lr_cnt, float scale, void* O,
                                                void* stream) {
    size_t need = 0;
    lsa_status s = lsa_attend_workspace_bytes(layout, cfg, batch, n_q, &need);
    if (s != LSA_OK) return s;
    if (need > kNoAllocScratchBytes) {
        char msg[200];
        snprintf(msg, sizeof(msg),
                 "lsa_sparse_attend_noalloc: this call needs %zu bytes of split-key scratch, the library holds %zu "
                 "(use lsa_sparse_attend with a workspace)",
                 need, kNoAllocScratchBytes);
        return lsa::set_error(LSA_ERR_WORKSPACE, msg);
    }
    void* ws = nullptr;
    if (need > 0) {
        ws = scratch_for_current_device();
        if (ws == nullptr) return LSA_ERR_HIP;
    }
    return lsa_sparse_attend(layout, cfg, Q, K, V, t_cap, T, q_pos, batch, n_q, lr_idx, lr_cnt, scale, O, ws,
                             need > 0 ? kNoAllocScratchBytes : 0, stream);
}
