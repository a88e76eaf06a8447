// Host-side launch interface between the C ABI (lsa_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lsa_common.hpp"

namespace lsa {

struct SelArgs {
    int32_t k;
    int32_t n_sinks;
    int32_t window;
    int32_t beam;
    int32_t H_q;
    int32_t G;
    int32_t H_kv;
    int64_t n_q;
    int64_t n_units;   // B * n_q * H_kv
};

struct SelectBuffers {
    void* qhat;
    float* tau;
    int* cnt;
    uint64_t* cand;
    int* fb_list;
    int* counters;
    float* scores;
    int64_t score_stride;
    int fb_slots;
};

struct AttArgs {
    int64_t n_q;
    int64_t n_units;
    int64_t t_cap;
    int32_t B, H_kv, H_q, G;
    int32_t n_sinks, window, n_blocks, k;
    int32_t splits;
    float scale;
    unsigned long long* arrive;   // splits > 1: per-unit arrival words (tag << 32 | count)
    uint32_t tag;                 // distinct per call
};

hipError_t launch_build(const CacheView& cv, const void* K, bool bf16, int64_t t_cap, int d, int B, int H_kv,
                        const void* W, hipStream_t st);
hipError_t launch_tree(const CacheView& cv, const int64_t* level_off, const int64_t* level_size, int B, int H_kv,
                       hipStream_t st);
hipError_t launch_qlatent(const void* Q, const void* W, bool bf16, int d, int64_t rows, void* qhat, int* counters,
                          void* zero, size_t zero_bytes, hipStream_t st);
hipError_t launch_select_fused(const CacheView& cv, bool bf16, const int64_t* q_pos, const SelArgs& sa, int B,
                               const SelectBuffers& sb, int32_t* lr_idx, int32_t* lr_cnt, hipStream_t st);
hipError_t launch_select_materialized(const CacheView& cv, bool bf16, const int64_t* q_pos, const SelArgs& sa,
                                      const SelectBuffers& sb, int32_t* lr_idx, int32_t* lr_cnt, hipStream_t st);
hipError_t launch_select_tree(const CacheView& cv, bool bf16, const int64_t* q_pos, const SelArgs& sa,
                              const SelectBuffers& sb, int32_t* lr_idx, int32_t* lr_cnt, hipStream_t st);
int attend_splits(int64_t n_units, int window, int k);
hipError_t launch_attend(const void* Q, const void* K, const void* V, const int64_t* q_pos, const int32_t* lr_idx,
                         const int32_t* lr_cnt, const AttArgs& aa, int D, bool bf16, void* O, float* part,
                         hipStream_t st);

}  // namespace lsa
