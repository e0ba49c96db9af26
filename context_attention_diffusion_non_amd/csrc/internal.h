// Internal launch interfaces of the cpattn kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cpattn {

// Epilogue of the attention kernel.
enum AttnEpilogue : int {
    EPI_STORE = 0,  // write the chunk's own (out, lse)
    EPI_MERGE = 1,  // LSE-merge the chunk's (out, lse) into an fp32 accumulator read from acc_in/lse_in
};

struct AttnArgs {
    const void* q;
    const void* k;
    const void* v;
    void* out;             // destination: out_fp32 ? float : bf16, [planes, Sq, D]
    float* lse_out;        // [planes, Sq]
    const float* acc_in;   // EPI_MERGE: fp32 accumulator [planes, Sq, D] (may equal out)
    const float* lse_in;   // EPI_MERGE: accumulator LSE [planes, Sq] (may equal lse_out)
    int64_t n_planes;      // B * H
    int64_t Sq;
    int64_t Skv;           // keys of this block (chunk length)
    int64_t kv_plane;      // elements between consecutive K/V planes (kv_ld * D)
    float scale_log2;      // softmax scale * log2(e)
    int mode;              // AttnEpilogue
    int out_fp32;          // 1: fp32 destination, 0: bf16
    int in_fp32;           // 1: q/k/v are fp32 (rounded to bf16 on staging)
    int d;                 // 64 or 128
};

hipError_t launch_attn_fwd(const AttnArgs& a, hipStream_t stream);

struct MergeArgs {
    float* acc_out;
    float* acc_lse;
    const void* blk_out;
    const float* blk_lse;
    int64_t rows;
    int64_t d;
    int blk_fp32;          // 1: blk_out fp32, 0: bf16
};

hipError_t launch_lse_merge(const MergeArgs& a, hipStream_t stream);

struct PermuteArgs {
    const void* in;
    void* out;
    int64_t B, S_local, H, d;
    int degree;
    int group;             // -1: all groups
    int direction;         // 0 seq->head, 1 head->seq
    int64_t elem_bytes;
};

hipError_t launch_ulysses_permute(const PermuteArgs& a, hipStream_t stream);

}  // namespace cpattn
