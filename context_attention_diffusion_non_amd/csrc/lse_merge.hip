// fp32 log-sum-exp merge of a partial attention result into an accumulator.
//
// Per row r (the log-sum-exp identity behind ContextParallelConfig's
// convert_to_fp32 ring numerics, "Parallelism" API page):
//   L = log(exp(La) + exp(Lb));  acc = exp(La - L) * acc + exp(Lb - L) * blk;  La = L
// A side whose LSE is -inf contributes exactly nothing (its output values are
// not read into the result), and two empty sides give 0 and -inf.
//
// HBM-bound: every byte is touched once, so the row data moves with
// non-temporal loads and stores.  Each thread merges float4 pieces;
// a wave covers whole rows (d is a power of two <= 256), so the in-place LSE
// update by the row's first lane cannot race with another wave reading it.
#include "internal.h"

#include <math.h>

namespace cpattn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

constexpr int NT = 256;
constexpr int UNR = 4;  // float4 pieces per thread
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ bool is_neg_inf(float x) { return __float_as_uint(x) == 0xff800000u; }

template <int BLK>
__global__ __launch_bounds__(NT) void lse_merge_kernel(MergeArgs a, int64_t n_items, int shift) {
    // shift = log2(d / 4): items per row is a power of two
    f32x4 acc[UNR], blk[UNR];
    float la[UNR], lb[UNR];
    int64_t item[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
        item[u] = ((int64_t)blockIdx.x * UNR + u) * NT + threadIdx.x;
        if (item[u] < n_items) {
            const int64_t row = item[u] >> shift;
            acc[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a.acc_out + item[u] * 4));
            if constexpr (BLK == DT_F32) {
                blk[u] = __builtin_nontemporal_load(
                    reinterpret_cast<const f32x4*>(static_cast<const float*>(a.blk_out) + item[u] * 4));
            } else if constexpr (BLK == DT_F16) {
                const f16x4 b = __builtin_nontemporal_load(
                    reinterpret_cast<const f16x4*>(static_cast<const _Float16*>(a.blk_out) + item[u] * 4));
                blk[u] = __builtin_convertvector(b, f32x4);
            } else {
                const bf16x4 b = __builtin_nontemporal_load(
                    reinterpret_cast<const bf16x4*>(static_cast<const __bf16*>(a.blk_out) + item[u] * 4));
                blk[u] = __builtin_convertvector(b, f32x4);
            }
            la[u] = a.acc_lse[row];
            lb[u] = a.blk_lse[row];
        }
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
        if (item[u] >= n_items) continue;
        const float mx = fmaxf(la[u], lb[u]);
        float wa = 0.f, wb = 0.f, lnew = -INFINITY;
        if (mx != -INFINITY) {
            const float ea = __builtin_amdgcn_exp2f((la[u] - mx) * kLog2e);
            const float eb = __builtin_amdgcn_exp2f((lb[u] - mx) * kLog2e);
            const float tot = ea + eb;
            const float it = 1.f / tot;
            wa = ea * it;
            wb = eb * it;
            lnew = mx + __builtin_amdgcn_logf(tot) * kLn2;
        }
        // An empty side (LSE = -inf, tested on its bits so the test survives
        // -fno-honor-nans) is selected out, never multiplied by 0: its values
        // may be anything, NaN included.
        f32x4 r = {0.f, 0.f, 0.f, 0.f};
        if (!is_neg_inf(la[u])) r = acc[u] * wa;
        if (!is_neg_inf(lb[u])) r = r + blk[u] * wb;
        __builtin_nontemporal_store(r, reinterpret_cast<f32x4*>(a.acc_out + item[u] * 4));
        if ((item[u] & ((1 << shift) - 1)) == 0) a.acc_lse[item[u] >> shift] = lnew;
    }
}

}  // namespace

hipError_t launch_lse_merge(const MergeArgs& a, hipStream_t stream) {
    if (a.rows <= 0) return hipSuccess;
    const int64_t per_row = a.d / 4;
    int shift = 0;
    while ((int64_t(1) << shift) < per_row) ++shift;
    const int64_t n_items = a.rows * per_row;
    const int64_t nblk = (n_items + (int64_t)NT * UNR - 1) / ((int64_t)NT * UNR);
    switch (a.blk_dtype) {
        case DT_F32:
            hipLaunchKernelGGL((lse_merge_kernel<DT_F32>), dim3((unsigned)nblk), dim3(NT), 0, stream, a, n_items, shift);
            break;
        case DT_F16:
            hipLaunchKernelGGL((lse_merge_kernel<DT_F16>), dim3((unsigned)nblk), dim3(NT), 0, stream, a, n_items, shift);
            break;
        case DT_BF16:
            hipLaunchKernelGGL((lse_merge_kernel<DT_BF16>), dim3((unsigned)nblk), dim3(NT), 0, stream, a, n_items, shift);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace cpattn
