// Internal launch interfaces of the cpattn kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cpattn {

// Element types of tensors crossing the kernels (same values as cpattn_dtype).
enum ElemType : int {
    DT_BF16 = 0,
    DT_F32 = 1,
    DT_F16 = 2,
};

// Epilogue of the attention kernel.
enum AttnEpilogue : int {
    EPI_STORE = 0,  // write the chunk's own (out, lse)
    EPI_MERGE = 1,  // LSE-merge the chunk's (out, lse) into the accumulator read from acc_in/lse_in
};

struct AttnArgs {
    const void* q;
    const void* k;
    const void* v;
    void* out;             // destination of element type out_dtype, [planes, Sq, D]
    float* lse_out;        // [planes, Sq]
    const void* acc_in;    // EPI_MERGE: accumulator [planes, Sq, D] of element type acc_dtype (may equal out)
    const float* lse_in;   // EPI_MERGE: accumulator LSE [planes, Sq] (may equal lse_out)
    int64_t n_planes;      // B * H
    int64_t Sq;
    int64_t Skv;           // keys of this block (chunk length)
    int64_t kv_plane;      // elements between consecutive K/V planes (kv_ld * D)
    float scale_log2;      // softmax scale * log2(e)
    int mode;              // AttnEpilogue
    int out_dtype;         // ElemType of out
    int in_dtype;          // ElemType of q/k/v (DT_F32 is rounded to bf16 on staging)
    int acc_dtype;         // ElemType of acc_in (DT_F32 unless the ring keeps partials in the output dtype)
    int d;                 // 64 or 128
};

hipError_t launch_attn_fwd(const AttnArgs& a, hipStream_t stream);

// One ring step in one launch (attn_ring_kernel + ring_fixup_kernel): whole
// query tiles in rounds of S workgroups, the leftover tiles cut into a head
// and a tail balanced over all S (see attn_fwd.hip).
constexpr int kRingMaxChunks = 128;  // non-empty chunks a launch can take
constexpr int kRingMinTiles = 8;     // fewest key tiles per workgroup
constexpr int kRingCUs = 256;        // MI355X compute units
// Waves resident per SIMD (registers and LDS allow 2 at d = 128 and 4 at
// d = 64), hence workgroups of NW waves per CU; 32 query rows per wave.  Both
// kinds of step run eight-wave workgroups (256 query rows, each K/V tile staged
// once for all of them: measured 7% faster than four-wave ones on the Mochi
// share); four-wave ones remain instantiated for the fallback rule below.
template <int D>
constexpr int kRingWavesPerSimd = D == 64 ? 4 : 2;
inline int ring_waves_per_simd(int64_t d) { return d == 64 ? kRingWavesPerSimd<64> : kRingWavesPerSimd<128>; }
// workgroups of NW waves resident on the chip
inline int ring_slots(int64_t d, int nw) { return kRingCUs * 4 * ring_waves_per_simd(d) / nw; }
// Waves per workgroup of a step that runs in rounds (its query tiles are 32 x that rows).
#ifndef CPATTN_RING_SPLIT_WAVES
#define CPATTN_RING_SPLIT_WAVES 8
#endif
constexpr int kRingSplitWaves = CPATTN_RING_SPLIT_WAVES;

// Workspace of a split ring step with G ranges: the fp32 pieces of cut query
// tiles ([2G, rows, d]), then their LSE ([2G, rows]) at a 256-byte offset.
constexpr size_t ring_align256(size_t x) { return (x + 255) & ~size_t(255); }
constexpr size_t ring_slot_lse_off(int64_t G, int64_t rows, int64_t d) {
    return ring_align256((size_t)(2 * G * rows * d) * 4);
}
constexpr size_t ring_slot_bytes(int64_t G, int64_t rows, int64_t d) {
    return ring_slot_lse_off(G, rows, d) + (size_t)(2 * G * rows) * 4;
}
// The most any one-launch step needs: 128-row slots for all ranges, either head dim.
constexpr size_t kRingScratchMax =
    ring_slot_bytes(kRingCUs * 4 * kRingWavesPerSimd<64> / kRingSplitWaves, 32 * kRingSplitWaves, 64) >
            ring_slot_bytes(kRingCUs * 4 * kRingWavesPerSimd<128> / kRingSplitWaves, 32 * kRingSplitWaves, 128)
        ? ring_slot_bytes(kRingCUs * 4 * kRingWavesPerSimd<64> / kRingSplitWaves, 32 * kRingSplitWaves, 64)
        : ring_slot_bytes(kRingCUs * 4 * kRingWavesPerSimd<128> / kRingSplitWaves, 32 * kRingSplitWaves, 128);

// The ring step (cpattn_ring_fwd's checks and launches) on caller-provided
// scratch of `bytes` bytes that the library allocated itself, for the
// allocation-free entry point: more than kRingMaxChunks chunks (whose per-chunk
// loop needs an accumulator of the problem's size) are refused.
int ring_fwd_on_scratch(const void* q, const void* k, const void* v, void* out, float* lse, int64_t B, int64_t H,
                        int64_t Sq, int64_t Skv, int64_t d, float scale, int ring_degree, const int64_t* chunk_lens,
                        void* scratch, size_t bytes, int in_dtype, int out_dtype, void* stream);
// Record a failed HIP call as the calling thread's last error; returns CPATTN_ERR_HIP.
int report_hip_error(hipError_t e, const char* what);

struct RingArgs {
    const void* q;
    const void* k;
    const void* v;
    void* out;             // [planes, Sq, D] of out_dtype
    float* lse_out;        // [planes, Sq]
    float* part_o;         // workspace: [2 * n_ranges, slot_rows, D] fp32 pieces of cut query tiles
    float* part_lse;       // workspace: [2 * n_ranges, slot_rows] their LSE, log2 units
    int64_t n_planes;      // B * H
    int64_t Sq;
    int64_t kv_plane;      // elements between consecutive K/V planes (Skv * D)
    int64_t slot_rows;     // rows per workspace slot: min(query rows per tile, Sq)
    int64_t tail_per;      // tail units (left * (T - head)) per tail range: tail_per, +1 for the first tail_rem
    int64_t tail_rem;
    int T;                 // key tiles per query tile, all chunks
    int nq;                // query tiles per plane
    int n_ranges;          // S: workgroups of the launch
    int rounds;            // R: full rounds of whole query tiles
    int left;              // L: query tiles after the rounds (< S)
    int head;              // key tiles of a leftover tile's head (0 .. T)
    int n_chunks;          // non-empty chunks
    int nw;                // waves per workgroup: 4, or 8 for a step of whole tiles in one round
    float scale_log2;
    int out_dtype;
    int in_dtype;
    int d;
    int chunk_tile0[kRingMaxChunks + 1];  // first key tile of each chunk; [n_chunks] = T
    int chunk_off[kRingMaxChunks];        // first key row of each chunk
    int chunk_len[kRingMaxChunks];        // keys of each chunk (> 0)
};

hipError_t launch_attn_ring(const RingArgs& a, hipStream_t stream);

struct MergeArgs {
    float* acc_out;
    float* acc_lse;
    const void* blk_out;
    const float* blk_lse;
    int64_t rows;
    int64_t d;
    int blk_dtype;         // ElemType of blk_out
};

hipError_t launch_lse_merge(const MergeArgs& a, hipStream_t stream);

struct PermuteArgs {
    const void* in;
    void* out;
    int64_t B, S_local, H, d;
    int degree;            // sequence shards P
    int group;             // head group to move, -1: all groups
    int direction;         // 0 seq->head, 1 head->seq
    int64_t elem_bytes;
    int groups;            // head groups G (H % G == 0); the Ulysses permute has G == P
    int rot;               // seq->head: output block r takes shard (r + rot) % P
};

hipError_t launch_ulysses_permute(const PermuteArgs& a, hipStream_t stream);

// Ulysses Anything regroup: uneven sequence shards and head groups.
constexpr int kAnyMaxDegree = 32;

struct AnyPermuteArgs {
    const void* in;
    void* out;
    int64_t B, H, d;
    int degree;                              // P
    const int64_t* seq_lens;                 // host, P entries (tokens of shard r)
    const int64_t* head_lens;                // host, P entries (heads of group g), sum H
    int group;                               // -1: all groups (stacked, group g at B * hoff_g * S * d)
    int direction;                           // 0 seq->head, 1 head->seq
    int64_t elem_bytes;
};

hipError_t launch_ulysses_anything_permute(const AnyPermuteArgs& a, hipStream_t stream);

}  // namespace cpattn
