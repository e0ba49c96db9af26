// C ABI of cpattn: argument validation, the ring driver and error reporting.
// Declarations and the contract of every entry point are in include/cpattn.h.
#include "cpattn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "internal.h"

#define CPATTN_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return status;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(CPATTN_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

static_assert((int)CPATTN_BF16 == (int)cpattn::DT_BF16 && (int)CPATTN_FP32 == (int)cpattn::DT_F32 &&
                  (int)CPATTN_FP16 == (int)cpattn::DT_F16,
              "cpattn_dtype and the kernels' element types must agree");

bool valid_dtype(int dt) { return dt == CPATTN_BF16 || dt == CPATTN_FP32 || dt == CPATTN_FP16; }
size_t dtype_bytes(int dt) { return dt == CPATTN_FP32 ? 4 : 2; }

// Byte ranges [p, p+n) and [q, q+m) intersect (empty ranges never do).
bool overlaps(const void* p, size_t n, const void* q, size_t m) {
    if (p == nullptr || q == nullptr || n == 0 || m == 0) return false;
    const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
    return a < b + m && b < a + n;
}

// a * b * ... without int64 overflow; false on overflow or a negative factor.
bool mul_ok(int64_t& acc, int64_t f) {
    if (f < 0) return false;
    if (f != 0 && acc > INT64_MAX / f) return false;
    acc *= f;
    return true;
}

constexpr int64_t kMaxBlocks = (int64_t(1) << 31) - 1;

float resolve_scale(float scale, int64_t d) {
    if (!(scale > 0.f) || std::isinf(scale)) return 1.0f / std::sqrt((float)d);
    return scale;
}

struct AttnCheck {
    size_t q_bytes, kv_bytes, out_bytes, lse_bytes;
};

// Shared checks of the attention entry points.
int check_attn(const void* q, const void* k, const void* v, const void* out, const void* lse, int64_t B, int64_t H,
               int64_t Sq, int64_t Skv, int64_t kv_ld, int64_t d, int in_dt, int out_dt, AttnCheck& c) {
    if (B < 1 || H < 1) return fail(CPATTN_ERR_SHAPE, "B and H must be >= 1 (got B=%lld H=%lld)", (long long)B, (long long)H);
    if (Sq < 0 || Skv < 0) return fail(CPATTN_ERR_SHAPE, "sequence lengths must be >= 0 (Sq=%lld Skv=%lld)", (long long)Sq, (long long)Skv);
    if (kv_ld < Skv) return fail(CPATTN_ERR_SHAPE, "kv_ld (%lld) must be >= Skv (%lld)", (long long)kv_ld, (long long)Skv);
    if (d != 64 && d != 128) return fail(CPATTN_ERR_SHAPE, "head dim d must be 64 or 128 (got %lld)", (long long)d);
    if (!valid_dtype(in_dt)) return fail(CPATTN_ERR_DTYPE, "unsupported input dtype %d", in_dt);
    if (!valid_dtype(out_dt)) return fail(CPATTN_ERR_DTYPE, "unsupported output dtype %d", out_dt);
    int64_t nq = B;
    int64_t nkv = B;
    int64_t nblk = B;
    if (!mul_ok(nq, H) || !mul_ok(nq, Sq) || !mul_ok(nq, d) || !mul_ok(nq, 4) || !mul_ok(nkv, H) ||
        !mul_ok(nkv, kv_ld) || !mul_ok(nkv, d) || !mul_ok(nkv, 4) || !mul_ok(nblk, H) || !mul_ok(nblk, (Sq + 127) / 128))
        return fail(CPATTN_ERR_SHAPE, "tensor sizes overflow");
    if (nblk > kMaxBlocks) return fail(CPATTN_ERR_SHAPE, "too many query tiles (%lld)", (long long)nblk);
    if (Skv > INT32_MAX - 64) return fail(CPATTN_ERR_SHAPE, "Skv too large (%lld)", (long long)Skv);
    c.q_bytes = (size_t)(B * H * Sq * d) * dtype_bytes(in_dt);
    // the last plane only reaches row Skv: a chunk passed in place ends inside its parent buffer
    c.kv_bytes = Skv > 0 ? (size_t)(((B * H - 1) * kv_ld + Skv) * d) * dtype_bytes(in_dt) : 0;
    c.out_bytes = (size_t)(B * H * Sq * d) * dtype_bytes(out_dt);
    c.lse_bytes = (size_t)(B * H * Sq) * 4;
    if (Sq > 0) {
        if (q == nullptr) return fail(CPATTN_ERR_NULL, "q is NULL");
        if (out == nullptr) return fail(CPATTN_ERR_NULL, "out is NULL");
        if (lse == nullptr) return fail(CPATTN_ERR_NULL, "lse is NULL");
    }
    if (Skv > 0 && Sq > 0) {
        if (k == nullptr) return fail(CPATTN_ERR_NULL, "k is NULL");
        if (v == nullptr) return fail(CPATTN_ERR_NULL, "v is NULL");
    }
    const void* ins[3] = {q, k, v};
    const size_t in_sz[3] = {c.q_bytes, c.kv_bytes, c.kv_bytes};
    for (int i = 0; i < 3; ++i) {
        if (overlaps(out, c.out_bytes, ins[i], in_sz[i]) || overlaps(lse, c.lse_bytes, ins[i], in_sz[i]))
            return fail(CPATTN_ERR_ALIAS, "out/lse overlap an input");
    }
    if (overlaps(out, c.out_bytes, lse, c.lse_bytes)) return fail(CPATTN_ERR_ALIAS, "out overlaps lse");
    return CPATTN_OK;
}

cpattn::AttnArgs make_args(const void* q, const void* k, const void* v, void* out, float* lse, int64_t B, int64_t H,
                           int64_t Sq, int64_t Skv, int64_t kv_ld, int64_t d, float scale, int in_dt, int out_dt) {
    cpattn::AttnArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.lse_out = lse;
    a.acc_in = nullptr;
    a.lse_in = nullptr;
    a.acc_dtype = cpattn::DT_F32;
    a.n_planes = B * H;
    a.Sq = Sq;
    a.Skv = Skv;
    a.kv_plane = kv_ld * d;
    a.scale_log2 = resolve_scale(scale, d) * 1.4426950408889634f;
    a.mode = cpattn::EPI_STORE;
    a.out_dtype = out_dt;
    a.in_dtype = in_dt;
    a.d = (int)d;
    return a;
}

// The ring loop after validation: chunk 0 stores its partial into the
// accumulator, later chunks LSE-merge into it in their epilogue, and the last
// one writes `out`.  The accumulator is fp32 (convert_to_fp32): the output
// itself when it is fp32 or when there is a single chunk, else `acc_ws`.  With
// partials_fp32 false it is `out` in the output dtype, rounded after every
// merge.  Chunks are `chunk_lens` (NULL: equal lengths).
int ring_launch(const void* q, const void* k, const void* v, void* out, float* lse, int64_t B, int64_t H, int64_t Sq,
                int64_t Skv, int64_t d, float scale, int ring_degree, const int64_t* chunk_lens, float* acc_ws,
                int in_dtype, int out_dtype, hipStream_t s, bool partials_fp32 = true) {
    const size_t esz = dtype_bytes(in_dtype);
    const bool acc_is_out = ring_degree == 1 || out_dtype == CPATTN_FP32 || !partials_fp32;
    void* acc = acc_is_out ? out : static_cast<void*>(acc_ws);
    const int acc_dt = acc_is_out ? out_dtype : (int)cpattn::DT_F32;
    int64_t off = 0;
    for (int c_i = 0; c_i < ring_degree; ++c_i) {
        const int64_t len = chunk_lens ? chunk_lens[c_i] : Skv / ring_degree;
        const char* kc = static_cast<const char*>(k) + (size_t)off * d * esz;
        const char* vc = static_cast<const char*>(v) + (size_t)off * d * esz;
        cpattn::AttnArgs a = make_args(q, kc, vc, nullptr, lse, B, H, Sq, len, Skv, d, scale, in_dtype, out_dtype);
        const bool last = c_i == ring_degree - 1;
        if (c_i == 0) {
            a.mode = cpattn::EPI_STORE;
        } else {
            a.mode = cpattn::EPI_MERGE;
            a.acc_in = acc;
            a.acc_dtype = acc_dt;
            a.lse_in = lse;
        }
        if (last) {
            a.out = out;
            a.out_dtype = out_dtype;
        } else {
            a.out = acc;
            a.out_dtype = acc_dt;
        }
        const hipError_t e = cpattn::launch_attn_fwd(a, s);
        if (e != hipSuccess) return hip_fail(e, "attention kernel launch (ring chunk)");
        off += len;
    }
    return CPATTN_OK;
}


size_t align256(size_t x) { return cpattn::ring_align256(x); }

size_t ring_slot_bytes(int64_t G, int64_t rows, int64_t d, size_t* lse_off) {
    if (lse_off) *lse_off = cpattn::ring_slot_lse_off(G, rows, d);
    return cpattn::ring_slot_bytes(G, rows, d);
}

// Workspace the ring step needs at most for these sizes (any chunking): the
// one-launch step's slots for its most ranges, or, past kRingMaxChunks
// chunks, the per-chunk loop's fp32 accumulator when the output is not fp32.
size_t ring_ws_bound(int64_t B, int64_t H, int64_t Sq, int64_t d, int ring_degree, int out_dtype) {
    if (ring_degree <= cpattn::kRingMaxChunks) {
        if (Sq == 0) return 0;
        // slots x rows is the same for four- and eight-wave workgroups
        const int64_t rows = 32 * cpattn::kRingSplitWaves;
        return ring_slot_bytes(cpattn::ring_slots(d, cpattn::kRingSplitWaves), Sq < rows ? Sq : rows, d, nullptr);
    }
    if (out_dtype == CPATTN_FP32) return 0;
    int64_t n = B;
    if (!mul_ok(n, H) || !mul_ok(n, Sq) || !mul_ok(n, d) || !mul_ok(n, 4)) return 0;
    return (size_t)n;
}

// Launch geometry of the one-launch ring step (valid, validated arguments).
struct RingPlan {
    cpattn::RingArgs a;
    size_t need;     // workspace bytes the launch writes (0: no range boundary cuts a query tile)
    size_t lse_off;
};

void ring_plan(RingPlan& p, const void* q, const void* k, const void* v, void* out, float* lse, int64_t B, int64_t H,
               int64_t Sq, int64_t Skv, int64_t d, float scale, int ring_degree, const int64_t* chunk_lens,
               int in_dtype, int out_dtype) {
    cpattn::RingArgs& a = p.a;
    a = cpattn::RingArgs{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.lse_out = lse;
    a.n_planes = B * H;
    a.Sq = Sq;
    a.kv_plane = Skv * d;
    a.scale_log2 = resolve_scale(scale, d) * 1.4426950408889634f;
    a.out_dtype = out_dtype;
    a.in_dtype = in_dtype;
    a.d = (int)d;
    int n = 0, T = 0;
    int64_t off = 0;
    for (int i = 0; i < ring_degree; ++i) {
        const int64_t len = chunk_lens ? chunk_lens[i] : Skv / ring_degree;
        if (len > 0) {
            a.chunk_off[n] = (int)off;
            a.chunk_len[n] = (int)len;
            a.chunk_tile0[n] = T;
            T += (int)((len + 63) / 64);
            ++n;
        }
        off += len;
    }
    a.chunk_tile0[n] = T;
    a.n_chunks = n;
    a.T = T;
    // Whole query tiles of 256 rows in one round of eight-wave workgroups when even
    // 128-row tiles would not fill a round of four-wave ones (the chip then stays at
    // its full clock with some CUs idle, which splitting tiles measured no faster);
    // else query tiles of 32 * kRingSplitWaves rows in rounds, the leftover ones split.
    const int64_t q4 = a.n_planes * ((Sq + 127) / 128), q8 = a.n_planes * ((Sq + 255) / 256);
    if (q4 <= cpattn::ring_slots(d, 4) && q8 <= cpattn::ring_slots(d, 8)) {
        a.nw = 8;
        a.nq = (int)((Sq + 255) / 256);
        a.n_ranges = (int)q8;
        a.rounds = 1;
        a.left = 0;
        a.head = 0;
        a.tail_per = 0;
        a.tail_rem = 0;
        a.slot_rows = Sq < 256 ? Sq : 256;
        p.need = 0;
        return;
    }
    a.nw = cpattn::kRingSplitWaves;
    const int rows = 32 * a.nw;
    a.nq = (int)((Sq + rows - 1) / rows);
    const int64_t Q = a.n_planes * a.nq;
    int64_t S = (Q * (int64_t)T + cpattn::kRingMinTiles - 1) / cpattn::kRingMinTiles;
    if (S > cpattn::ring_slots(d, a.nw)) S = cpattn::ring_slots(d, a.nw);
    if (S < 1) S = 1;
    a.n_ranges = (int)S;
    a.rounds = (int)(Q / S);
    a.left = (int)(Q % S);
    const int64_t L = a.left;
    int64_t Hd = L > 0 ? (2 * L * T + S) / (2 * S) : 0;  // round(L T / S)
    if (Hd > T) Hd = T;
    a.head = (int)Hd;
    const int64_t tail_units = L * (T - Hd), tail_ranges = S - L;
    a.tail_per = tail_units / tail_ranges;
    a.tail_rem = tail_units % tail_ranges;
    a.slot_rows = Sq < rows ? Sq : rows;
    // pieces go to the workspace when a leftover tile is cut: heads short of T, or
    // (no heads) a range boundary inside a tail
    bool split = L > 0 && Hd > 0 && Hd < T;
    if (L > 0 && Hd == 0) {
        for (int64_t t = 1; t < tail_ranges && !split; ++t)
            split = (t * a.tail_per + (t < a.tail_rem ? t : a.tail_rem)) % T != 0;
    }
    p.need = split ? ring_slot_bytes(S, a.slot_rows, d, &p.lse_off) : 0;
}

}  // namespace

CPATTN_EXPORT int cpattn_version(void) { return 110; }

CPATTN_EXPORT const char* cpattn_last_error(void) { return g_last_error; }

CPATTN_EXPORT const char* cpattn_status_string(int status) {
    switch (status) {
        case CPATTN_OK: return "ok";
        case CPATTN_ERR_NULL: return "null pointer";
        case CPATTN_ERR_SHAPE: return "invalid shape";
        case CPATTN_ERR_DEGREE: return "invalid degree";
        case CPATTN_ERR_INDIVISIBLE: return "size not divisible by degree";
        case CPATTN_ERR_CHUNKS: return "invalid chunk lengths";
        case CPATTN_ERR_DTYPE: return "unsupported dtype";
        case CPATTN_ERR_WORKSPACE: return "workspace too small";
        case CPATTN_ERR_ALIAS: return "output overlaps input";
        case CPATTN_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

CPATTN_EXPORT int cpattn_block_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int64_t B,
                                   int64_t H, int64_t Sq, int64_t Skv, int64_t kv_ld, int64_t d, float scale,
                                   int in_dtype, int out_dtype, void* stream) {
    AttnCheck c;
    const int st = check_attn(q, k, v, out, lse, B, H, Sq, Skv, kv_ld, d, in_dtype, out_dtype, c);
    if (st != CPATTN_OK) return st;
    if (Sq == 0) return CPATTN_OK;
    cpattn::AttnArgs a = make_args(q, k, v, out, lse, B, H, Sq, Skv, kv_ld, d, scale, in_dtype, out_dtype);
    const hipError_t e = cpattn::launch_attn_fwd(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "attention kernel launch");
    return CPATTN_OK;
}

CPATTN_EXPORT int cpattn_lse_merge(float* acc_out, float* acc_lse, const void* blk_out, const float* blk_lse,
                                   int64_t rows, int64_t d, int blk_dtype, void* stream) {
    if (rows < 0) return fail(CPATTN_ERR_SHAPE, "rows must be >= 0 (got %lld)", (long long)rows);
    if (d < 4 || d > 256 || (d & (d - 1)) != 0)
        return fail(CPATTN_ERR_SHAPE, "d must be a power of two in [4, 256] (got %lld)", (long long)d);
    if (!valid_dtype(blk_dtype)) return fail(CPATTN_ERR_DTYPE, "unsupported partial dtype %d", blk_dtype);
    if (rows == 0) return CPATTN_OK;
    if (!acc_out || !acc_lse || !blk_out || !blk_lse) return fail(CPATTN_ERR_NULL, "a merge pointer is NULL");
    int64_t n = rows;
    if (!mul_ok(n, d) || !mul_ok(n, 4)) return fail(CPATTN_ERR_SHAPE, "merge size overflows");
    const size_t acc_b = (size_t)(rows * d) * 4, blk_b = (size_t)(rows * d) * dtype_bytes(blk_dtype);
    const size_t lse_b = (size_t)rows * 4;
    if (overlaps(blk_out, blk_b, acc_out, acc_b) || overlaps(blk_out, blk_b, acc_lse, lse_b) ||
        overlaps(blk_lse, lse_b, acc_out, acc_b) || overlaps(blk_lse, lse_b, acc_lse, lse_b) ||
        overlaps(acc_out, acc_b, acc_lse, lse_b))
        return fail(CPATTN_ERR_ALIAS, "merge operands overlap");
    if ((rows * d / 4 + 1023) / 1024 > kMaxBlocks) return fail(CPATTN_ERR_SHAPE, "merge too large");
    cpattn::MergeArgs a{acc_out, acc_lse, blk_out, blk_lse, rows, d, blk_dtype};
    const hipError_t e = cpattn::launch_lse_merge(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "merge kernel launch");
    return CPATTN_OK;
}

CPATTN_EXPORT size_t cpattn_ring_fwd_workspace_bytes(int64_t B, int64_t H, int64_t Sq, int64_t d, int ring_degree,
                                                     int out_dtype) {
    if (B < 1 || H < 1 || Sq < 0 || d < 1 || d > 4096 || ring_degree < 1) return 0;
    return ring_ws_bound(B, H, Sq, d, ring_degree, out_dtype);
}

namespace {

int ring_fwd_impl(const void* q, const void* k, const void* v, void* out, float* lse, int64_t B, int64_t H,
                  int64_t Sq, int64_t Skv, int64_t d, float scale, int ring_degree, const int64_t* chunk_lens,
                  bool partials_fp32, void* workspace, size_t workspace_bytes, int in_dtype, int out_dtype,
                  void* stream) {
    if (ring_degree < 1) return fail(CPATTN_ERR_DEGREE, "ring_degree must be >= 1 (got %d)", ring_degree);
    AttnCheck c;
    int st = check_attn(q, k, v, out, lse, B, H, Sq, Skv, Skv, d, in_dtype, out_dtype, c);
    if (st != CPATTN_OK) return st;
    // chunk geometry (host side, no device sync)
    if (chunk_lens == nullptr) {
        if (Skv % ring_degree != 0)
            return fail(CPATTN_ERR_INDIVISIBLE, "Skv=%lld is not divisible by ring_degree=%d; pass chunk_lens",
                        (long long)Skv, ring_degree);
    } else {
        int64_t sum = 0;
        for (int i = 0; i < ring_degree; ++i) {
            if (chunk_lens[i] < 0) return fail(CPATTN_ERR_CHUNKS, "chunk_lens[%d] = %lld < 0", i, (long long)chunk_lens[i]);
            // compared before adding, so no sum of lengths can overflow and wrap back to Skv
            if (chunk_lens[i] > Skv - sum)
                return fail(CPATTN_ERR_CHUNKS, "chunk lengths exceed Skv=%lld at chunk %d", (long long)Skv, i);
            sum += chunk_lens[i];
        }
        if (sum != Skv) return fail(CPATTN_ERR_CHUNKS, "chunk lengths do not sum to Skv=%lld", (long long)Skv);
    }
    // convert_to_fp32 with at most kRingMaxChunks chunks: the whole step in one launch
    // (plus the merge of split query tiles); otherwise one launch per chunk.
    // (No keys at all: one launch writes out = 0, lse = -inf, and no workspace is used.)
    const bool one_launch = partials_fp32 && ring_degree <= cpattn::kRingMaxChunks && Skv > 0;
    RingPlan plan;
    size_t need = 0;
    if (one_launch) {
        ring_plan(plan, q, k, v, out, lse, B, H, Sq, Skv, d, scale, ring_degree, chunk_lens, in_dtype, out_dtype);
        need = plan.need;
    } else if (partials_fp32 && Skv > 0 && ring_degree > 1 && out_dtype != CPATTN_FP32) {
        need = (size_t)(B * H * Sq * d) * 4;  // the per-chunk loop's fp32 accumulator (sizes checked above)
    }
    if (need > 0) {
        if (workspace == nullptr || workspace_bytes < need)
            return fail(CPATTN_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
        if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
            return fail(CPATTN_ERR_WORKSPACE, "workspace must be 256-byte aligned");
        const void* ins[3] = {q, k, v};
        const size_t in_sz[3] = {c.q_bytes, c.kv_bytes, c.kv_bytes};
        for (int i = 0; i < 3; ++i)
            if (overlaps(workspace, need, ins[i], in_sz[i])) return fail(CPATTN_ERR_ALIAS, "workspace overlaps an input");
        if (overlaps(workspace, need, out, c.out_bytes) || overlaps(workspace, need, lse, c.lse_bytes))
            return fail(CPATTN_ERR_ALIAS, "workspace overlaps an output");
    }
    if (Sq == 0) return CPATTN_OK;

    if (Skv == 0) {
        const cpattn::AttnArgs a = make_args(q, k, v, out, lse, B, H, Sq, 0, 0, d, scale, in_dtype, out_dtype);
        const hipError_t e = cpattn::launch_attn_fwd(a, static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return hip_fail(e, "attention kernel launch (no keys)");
        return CPATTN_OK;
    }
    if (one_launch) {
        plan.a.part_o = static_cast<float*>(workspace);
        plan.a.part_lse = need > 0 ? reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.lse_off) : nullptr;
        const hipError_t e = cpattn::launch_attn_ring(plan.a, static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return hip_fail(e, "ring step launch");
        return CPATTN_OK;
    }
    return ring_launch(q, k, v, out, lse, B, H, Sq, Skv, d, scale, ring_degree, chunk_lens,
                       static_cast<float*>(workspace), in_dtype, out_dtype, static_cast<hipStream_t>(stream),
                       partials_fp32);
}

}  // namespace

namespace cpattn {

int ring_fwd_on_scratch(const void* q, const void* k, const void* v, void* out, float* lse, int64_t B, int64_t H,
                        int64_t Sq, int64_t Skv, int64_t d, float scale, int ring_degree, const int64_t* chunk_lens,
                        void* scratch, size_t bytes, int in_dtype, int out_dtype, void* stream) {
    if (ring_degree > kRingMaxChunks)
        return fail(CPATTN_ERR_DEGREE, "the allocation-free ring step takes at most %d chunks (got %d)", kRingMaxChunks,
                    ring_degree);
    return ring_fwd_impl(q, k, v, out, lse, B, H, Sq, Skv, d, scale, ring_degree, chunk_lens, true, scratch, bytes,
                         in_dtype, out_dtype, stream);
}

int report_hip_error(hipError_t e, const char* what) { return hip_fail(e, what); }

}  // namespace cpattn

CPATTN_EXPORT int cpattn_ring_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int64_t B,
                                  int64_t H, int64_t Sq, int64_t Skv, int64_t d, float scale, int ring_degree,
                                  const int64_t* chunk_lens, void* workspace, size_t workspace_bytes, int in_dtype,
                                  int out_dtype, void* stream) {
    return ring_fwd_impl(q, k, v, out, lse, B, H, Sq, Skv, d, scale, ring_degree, chunk_lens, true, workspace,
                         workspace_bytes, in_dtype, out_dtype, stream);
}

CPATTN_EXPORT int cpattn_ring_fwd_cfg(const void* q, const void* k, const void* v, void* out, float* lse, int64_t B,
                                      int64_t H, int64_t Sq, int64_t Skv, int64_t d, float scale, int ring_degree,
                                      const int64_t* chunk_lens, int convert_to_fp32, void* workspace,
                                      size_t workspace_bytes, int in_dtype, int out_dtype, void* stream) {
    return ring_fwd_impl(q, k, v, out, lse, B, H, Sq, Skv, d, scale, ring_degree, chunk_lens, convert_to_fp32 != 0,
                         workspace, workspace_bytes, in_dtype, out_dtype, stream);
}

CPATTN_EXPORT int cpattn_ulysses_permute(const void* in, void* out, int64_t B, int64_t S_local, int64_t H, int64_t d,
                                         int degree, int group, int direction, int64_t elem_bytes, void* stream) {
    if (degree < 1 || degree > 65535) return fail(CPATTN_ERR_DEGREE, "degree must lie in [1, 65535] (got %d)", degree);
    if (group < -1 || group >= degree) return fail(CPATTN_ERR_DEGREE, "group %d outside [-1, %d)", group, degree);
    if (direction != 0 && direction != 1) return fail(CPATTN_ERR_DTYPE, "direction must be 0 or 1 (got %d)", direction);
    if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4 && elem_bytes != 8)
        return fail(CPATTN_ERR_DTYPE, "elem_bytes must be 1, 2, 4 or 8 (got %lld)", (long long)elem_bytes);
    if (B < 1 || H < 1 || d < 1 || S_local < 0) return fail(CPATTN_ERR_SHAPE, "invalid permute shape");
    if (H % degree != 0) return fail(CPATTN_ERR_INDIVISIBLE, "H=%lld is not divisible by degree=%d", (long long)H, degree);
    int64_t n = degree;
    if (!mul_ok(n, B) || !mul_ok(n, S_local) || !mul_ok(n, H) || !mul_ok(n, d) || !mul_ok(n, elem_bytes))
        return fail(CPATTN_ERR_SHAPE, "permute size overflows");
    const int64_t groups = group < 0 ? degree : 1;
    const size_t seq_bytes = (size_t)n;                              // [P, B, S_loc, H, d]
    const size_t head_bytes = (size_t)(n / degree) * (size_t)groups;  // [G, B, H/P, S, d]
    if (S_local == 0) return CPATTN_OK;
    if (!in || !out) return fail(CPATTN_ERR_NULL, "in/out is NULL");
    const size_t in_b = direction == 0 ? seq_bytes : head_bytes;
    const size_t out_b = direction == 0 ? head_bytes : seq_bytes;
    if (overlaps(in, in_b, out, out_b)) return fail(CPATTN_ERR_ALIAS, "out overlaps in");
    int64_t row_bytes = d * elem_bytes;
    int U = 16;
    while (U > 1 && row_bytes % U != 0) U >>= 1;
    if ((B * S_local * (H / degree) * (row_bytes / U)) >= (int64_t(1) << 31))
        return fail(CPATTN_ERR_SHAPE, "one (rank, group) slice exceeds 2^31 copy units");
    cpattn::PermuteArgs a{in, out, B, S_local, H, d, degree, group, direction, elem_bytes, degree, 0};
    const hipError_t e = cpattn::launch_ulysses_permute(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "permute kernel launch");
    return CPATTN_OK;
}

namespace {

// Workspace layout of cpattn_unified_fwd: the regrouped q (the rank's Ulysses
// group's tokens, its head group), k and v (every token of the grid, its head
// group, in its ring order) and the ring's fp32 accumulator; 256-byte aligned.
struct UnifiedPlan {
    int64_t hq, s_seg, s_all;
    size_t q_off, k_off, v_off, acc_off, total;
    bool ok;
};


UnifiedPlan unified_plan(int64_t B, int64_t S_local, int64_t H, int64_t d, int R, int U, int in_dtype, int out_dtype) {
    UnifiedPlan p{};
    p.ok = false;
    if (B < 1 || H < 1 || S_local < 0 || d < 1 || R < 1 || U < 1 || H % U != 0) return p;
    if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return p;
    p.hq = H / U;
    int64_t seg = S_local, all = S_local;
    if (!mul_ok(seg, U) || !mul_ok(all, U) || !mul_ok(all, R)) return p;
    p.s_seg = seg;
    p.s_all = all;
    int64_t qn = B, kn = B, an = B;
    if (!mul_ok(qn, p.hq) || !mul_ok(qn, seg) || !mul_ok(qn, d) || !mul_ok(qn, (int64_t)dtype_bytes(in_dtype)) ||
        !mul_ok(kn, p.hq) || !mul_ok(kn, all) || !mul_ok(kn, d) || !mul_ok(kn, (int64_t)dtype_bytes(in_dtype)) ||
        !mul_ok(an, p.hq) || !mul_ok(an, seg) || !mul_ok(an, d) || !mul_ok(an, 4))
        return p;
    // the ring step's own workspace (pieces of split query tiles, or the per-chunk fp32 accumulator)
    const size_t ring_ws = ring_ws_bound(B, p.hq, seg, d, R, out_dtype);
    p.q_off = 0;
    p.k_off = align256((size_t)qn);
    p.v_off = p.k_off + align256((size_t)kn);
    p.acc_off = p.v_off + align256((size_t)kn);
    p.total = p.acc_off + align256(ring_ws);
    p.ok = true;
    return p;
}

}  // namespace

CPATTN_EXPORT size_t cpattn_unified_fwd_workspace_bytes(int64_t B, int64_t S_local, int64_t H, int64_t d,
                                                        int ring_degree, int ulysses_degree, int in_dtype,
                                                        int out_dtype) {
    const UnifiedPlan p = unified_plan(B, S_local, H, d, ring_degree, ulysses_degree, in_dtype, out_dtype);
    return p.ok ? p.total : 0;
}

CPATTN_EXPORT int cpattn_unified_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int64_t B,
                                     int64_t S_local, int64_t H, int64_t d, float scale, int ring_degree,
                                     int ulysses_degree, int ring_rank, int ulysses_rank, void* workspace,
                                     size_t workspace_bytes, int in_dtype, int out_dtype, void* stream) {
    const int R = ring_degree, U = ulysses_degree;
    if (R < 1 || U < 1 || (int64_t)R * U > 65535)
        return fail(CPATTN_ERR_DEGREE, "ring_degree=%d, ulysses_degree=%d: each >= 1, product <= 65535", R, U);
    if (ring_rank < 0 || ring_rank >= R || ulysses_rank < 0 || ulysses_rank >= U)
        return fail(CPATTN_ERR_DEGREE, "rank (%d, %d) outside the %d x %d grid", ring_rank, ulysses_rank, R, U);
    if (B < 1 || H < 1 || S_local < 0) return fail(CPATTN_ERR_SHAPE, "invalid unified shape");
    if (d != 64 && d != 128) return fail(CPATTN_ERR_SHAPE, "head dim d must be 64 or 128 (got %lld)", (long long)d);
    if (H % U != 0) return fail(CPATTN_ERR_INDIVISIBLE, "H=%lld is not divisible by ulysses_degree=%d", (long long)H, U);
    if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return fail(CPATTN_ERR_DTYPE, "unsupported dtype");
    const UnifiedPlan p = unified_plan(B, S_local, H, d, R, U, in_dtype, out_dtype);
    if (!p.ok) return fail(CPATTN_ERR_SHAPE, "unified sizes overflow");
    const int64_t W = (int64_t)R * U;
    int64_t shard_bytes = W;
    if (!mul_ok(shard_bytes, B) || !mul_ok(shard_bytes, S_local) || !mul_ok(shard_bytes, H) || !mul_ok(shard_bytes, d) ||
        !mul_ok(shard_bytes, (int64_t)dtype_bytes(in_dtype)))
        return fail(CPATTN_ERR_SHAPE, "unified sizes overflow");
    const int64_t row_bytes = d * (int64_t)dtype_bytes(in_dtype);
    if (B * S_local * p.hq * (row_bytes / 16) >= (int64_t(1) << 31))
        return fail(CPATTN_ERR_SHAPE, "one (shard, group) slice exceeds 2^31 copy units");
    if (S_local == 0) return CPATTN_OK;
    if (!q || !k || !v || !out || !lse) return fail(CPATTN_ERR_NULL, "a unified pointer is NULL");
    if (workspace == nullptr || workspace_bytes < p.total)
        return fail(CPATTN_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", p.total, workspace_bytes);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
        return fail(CPATTN_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    char* ws = static_cast<char*>(workspace);
    const void* ins[3] = {q, k, v};
    for (int i = 0; i < 3; ++i)
        if (overlaps(workspace, p.total, ins[i], (size_t)shard_bytes)) return fail(CPATTN_ERR_ALIAS, "workspace overlaps an input");
    // the regrouped tensors play q, k, v for the attention checks (sizes, out/lse aliasing)
    AttnCheck c;
    int st = check_attn(ws + p.q_off, ws + p.k_off, ws + p.v_off, out, lse, B, p.hq, p.s_seg, p.s_all, p.s_all, d,
                        in_dtype, out_dtype, c);
    if (st != CPATTN_OK) return st;
    for (int i = 0; i < 3; ++i)
        if (overlaps(out, c.out_bytes, ins[i], (size_t)shard_bytes) || overlaps(lse, c.lse_bytes, ins[i], (size_t)shard_bytes))
            return fail(CPATTN_ERR_ALIAS, "out/lse overlap an input");
    if (p.total > p.acc_off && (overlaps(ws + p.acc_off, p.total - p.acc_off, out, c.out_bytes) ||
                                overlaps(ws + p.acc_off, p.total - p.acc_off, lse, c.lse_bytes)))
        return fail(CPATTN_ERR_ALIAS, "workspace overlaps an output");

    const hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t eb = (int64_t)dtype_bytes(in_dtype);
    // q: the U shards of the rank's Ulysses group -> every token of its segment, head group ulysses_rank
    const char* q_grp = static_cast<const char*>(q) + (size_t)ring_rank * U * B * S_local * H * d * eb;
    cpattn::PermuteArgs pq{q_grp, ws + p.q_off, B, S_local, H, d, U, ulysses_rank, 0, eb, U, 0};
    // k, v: all W shards -> every token, head group ulysses_rank, segments in ring order from the rank's own
    cpattn::PermuteArgs pk{k, ws + p.k_off, B, S_local, H, d, (int)W, ulysses_rank, 0, eb, U, ring_rank * U};
    cpattn::PermuteArgs pv{v, ws + p.v_off, B, S_local, H, d, (int)W, ulysses_rank, 0, eb, U, ring_rank * U};
    const cpattn::PermuteArgs* perms[3] = {&pq, &pk, &pv};
    for (int i = 0; i < 3; ++i) {
        const hipError_t e = cpattn::launch_ulysses_permute(*perms[i], s);
        if (e != hipSuccess) return hip_fail(e, "unified regroup launch");
    }
    if (R <= cpattn::kRingMaxChunks) {
        RingPlan rp;
        ring_plan(rp, ws + p.q_off, ws + p.k_off, ws + p.v_off, out, lse, B, p.hq, p.s_seg, p.s_all, d, scale, R,
                  nullptr, in_dtype, out_dtype);
        rp.a.part_o = reinterpret_cast<float*>(ws + p.acc_off);
        rp.a.part_lse = reinterpret_cast<float*>(ws + p.acc_off + rp.lse_off);
        const hipError_t e = cpattn::launch_attn_ring(rp.a, s);
        if (e != hipSuccess) return hip_fail(e, "unified ring step launch");
        return CPATTN_OK;
    }
    return ring_launch(ws + p.q_off, ws + p.k_off, ws + p.v_off, out, lse, B, p.hq, p.s_seg, p.s_all, d, scale, R,
                       nullptr, reinterpret_cast<float*>(ws + p.acc_off), in_dtype, out_dtype, s);
}

CPATTN_EXPORT int cpattn_ulysses_anything_permute(const void* in, void* out, int64_t B, int64_t H, int64_t d,
                                                  int degree, const int64_t* seq_lens, const int64_t* head_lens,
                                                  int group, int direction, int64_t elem_bytes, void* stream) {
    if (degree < 1 || degree > cpattn::kAnyMaxDegree)
        return fail(CPATTN_ERR_DEGREE, "degree must lie in [1, %d] (got %d)", cpattn::kAnyMaxDegree, degree);
    if (group < -1 || group >= degree) return fail(CPATTN_ERR_DEGREE, "group %d outside [-1, %d)", group, degree);
    if (direction != 0 && direction != 1) return fail(CPATTN_ERR_DTYPE, "direction must be 0 or 1 (got %d)", direction);
    if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4 && elem_bytes != 8)
        return fail(CPATTN_ERR_DTYPE, "elem_bytes must be 1, 2, 4 or 8 (got %lld)", (long long)elem_bytes);
    if (B < 1 || H < 1 || d < 1) return fail(CPATTN_ERR_SHAPE, "invalid permute shape");
    if (seq_lens == nullptr || head_lens == nullptr) return fail(CPATTN_ERR_NULL, "seq_lens and head_lens are required");
    int64_t S = 0, hsum = 0;
    for (int i = 0; i < degree; ++i) {
        if (seq_lens[i] < 0 || head_lens[i] < 0)
            return fail(CPATTN_ERR_CHUNKS, "shard %d: negative length or head count", i);
        if (seq_lens[i] >= (int64_t(1) << 31) || head_lens[i] >= (int64_t(1) << 31))
            return fail(CPATTN_ERR_SHAPE, "shard %d too large", i);
        S += seq_lens[i];
        hsum += head_lens[i];
    }
    if (hsum != H) return fail(CPATTN_ERR_CHUNKS, "head counts sum to %lld, not H=%lld", (long long)hsum, (long long)H);
    int64_t n = B;
    if (!mul_ok(n, S) || !mul_ok(n, H) || !mul_ok(n, d) || !mul_ok(n, elem_bytes))
        return fail(CPATTN_ERR_SHAPE, "permute size overflows");
    int64_t max_s = 0;
    for (int i = 0; i < degree; ++i) max_s = seq_lens[i] > max_s ? seq_lens[i] : max_s;
    int64_t row_bytes = d * elem_bytes, U = 16;
    while (U > 1 && row_bytes % U != 0) U >>= 1;
    for (int i = 0; i < degree; ++i) {
        int64_t units = B;
        if (!mul_ok(units, max_s) || !mul_ok(units, head_lens[i]) || !mul_ok(units, row_bytes / U) ||
            units >= (int64_t(1) << 31))
            return fail(CPATTN_ERR_SHAPE, "one (shard, group) slice exceeds 2^31 copy units");
    }
    const size_t seq_bytes = (size_t)n;  // packed shards [B, s_r, H, d]
    const size_t head_bytes = group < 0 ? (size_t)n : (size_t)(B * head_lens[group] * S * d * elem_bytes);
    const size_t in_b = direction == 0 ? seq_bytes : head_bytes;
    const size_t out_b = direction == 0 ? head_bytes : seq_bytes;
    if (in_b == 0 || out_b == 0) return CPATTN_OK;  // no tokens, or a group without heads: nothing to move
    if (!in || !out) return fail(CPATTN_ERR_NULL, "in/out is NULL");
    if (overlaps(in, in_b, out, out_b)) return fail(CPATTN_ERR_ALIAS, "out overlaps in");
    cpattn::AnyPermuteArgs a{in, out, B, H, d, degree, seq_lens, head_lens, group, direction, elem_bytes};
    const hipError_t e = cpattn::launch_ulysses_anything_permute(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "permute kernel launch");
    return CPATTN_OK;
}
