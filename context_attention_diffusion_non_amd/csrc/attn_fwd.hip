// Attention forward of one query shard against one K/V block on gfx950.
//
// Computes, per (batch, head) plane and query row i,
//   out_i = sum_j softmax_j(scale * q_i . k_j) v_j,   lse_i = log sum_j exp(scale * q_i . k_j)
// -- the per-chunk step of ring attention ("Context parallelism" page, Ring
// Attention; ContextParallelConfig.ring_degree on the "Parallelism" API page)
// with the unmasked, non-causal scaled_dot_product_attention semantics of the
// ParaAttention README example.  In EPI_MERGE mode the chunk's (out, lse) is
// folded into an fp32 accumulator by the log-sum-exp identity in the epilogue
// (the convert_to_fp32 ring numerics), so the partial never round-trips HBM.
//
// Design (one workgroup = NW waves x 32 query rows of one plane; NW = 4, two
// workgroups per CU, or NW = 8, one per CU, when a launch fits the chip in one
// round -- the per-row arithmetic is the same either way):
//   * Everything is computed transposed: S^T = K Q^T and O^T = V^T P^T with
//     v_mfma_f32_32x32x16_bf16 (or its f16 twin for fp16 inputs, where P is
//     rounded to fp16 instead of bf16).  In the 32x32 accumulator layout a lane then
//     owns one query column and 16 of every 32 keys, so the row max / row sum
//     need one cross-half exchange (v_permlane32_swap) and the per-query
//     rescale of O is lane-local.
//   * Q stays in VGPRs as MFMA B fragments for the whole kernel.
//   * K and V tiles (64 keys) go global -> LDS directly (LDS DMA), row-major
//     with an XOR swizzle of 16-byte units per row.  K fragments are plain
//     16-byte LDS reads; V^T fragments come from two transposing LDS reads
//     (ds_read_b64_tr_b16), so no register staging or VALU transposes.  Two
//     LDS stages: the next tile's DMA runs under the current tile's math.
//   * Softmax in base 2 with scale*log2(e) folded into one FMA per score; the
//     running max used as the exponent base is only moved when a tile's max
//     exceeds it by more than 2^8, which keeps the O rescale off the common
//     path while every exp2 stays <= 256 (exact in the final O/l).
//   * Workgroup ids are remapped so each XCD (blocks go round-robin over the 8
//     XCDs) works on a contiguous range of (plane, query-tile) pairs and the
//     K/V of a plane stays in that XCD's L2.
#include "internal.h"

#include <math.h>

#include <type_traits>

namespace cpattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))

constexpr int BN = 64;   // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kSlack = 8.0f;  // log2 units a stale exponent base may lag the true max

// NW waves per workgroup, 32 query rows each.
template <int D, int NW>
struct Cfg {
    static constexpr int BM = 32 * NW;          // query rows per workgroup
    static constexpr int NT = 64 * NW;          // threads per workgroup
    static constexpr int RB = D * 2;            // LDS bytes per K or V row (bf16)
    static constexpr int UPR = D / 8;           // 16-byte units per row
    static constexpr int TILE = BN * RB;        // bytes of one K (or V) tile
    static constexpr int LDS = 4 * TILE;        // K stage 0 | K stage 1 | V stage 0 | V stage 1
    static constexpr int CHUNKS = TILE / 1024;  // 1 KB DMA chunks per tile
    static constexpr int CPW = CHUNKS / NW;     // chunks per wave
    static constexpr int NK = D / 16;           // k-steps of the S^T product
    static constexpr int NDB = D / 32;          // 32-row blocks of O^T
    static_assert(CHUNKS % NW == 0, "tile split over the waves");
    static_assert(LDS <= 65536, "stage offsets must fit the 16-bit LDS immediate");
};

// XOR swizzles of the 16-byte units of a row (rows are unpadded).
// K: a 16-byte read of 16 consecutive rows at one logical unit hits 16 distinct
//    bank groups.  V: a transposing 8-byte read over 4 rows x 64 bytes (half a
//    wave) hits distinct bank groups.
template <int D>
__device__ __forceinline__ int k_unit(int row, int u) {
    return D == 128 ? (u ^ (row & 15)) : (u ^ ((row >> 1) & 7));
}
template <int D>
__device__ __forceinline__ int v_unit(int row, int u) {
    return D == 128 ? (u ^ ((row & 3) << 2)) : (u ^ (((row >> 1) & 1) << 2));
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// Value from lane (lane ^ 32) combined with the own value.
__device__ __forceinline__ float pair_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 16-bit operand element of the MFMA path for an input element type: fp16
// inputs run on the f16 MFMA, bf16 and fp32 inputs on the bf16 one.
template <int IN>
struct Op {
    typedef __bf16 T8 __attribute__((ext_vector_type(8)));
};
template <>
struct Op<DT_F16> {
    typedef _Float16 T8 __attribute__((ext_vector_type(8)));
};

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32x32x16(f16x8 a, f16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 cvt8_f32_bf16(f32x4 a, f32x4 b) {
    f32x8 f = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    bf16x8 h = __builtin_convertvector(f, bf16x8);
    return __builtin_bit_cast(u32x4, h);
}

// 8 consecutive elements of a row as 16-bit operand bits: fp32 buffers are
// rounded to bf16, bf16 and fp16 buffers are taken as they are.
template <bool F32>
__device__ __forceinline__ u32x4 load8(const void* base, int64_t elem) {
    if constexpr (F32) {
        const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + elem);
        return cvt8_f32_bf16(p[0], p[1]);
    } else {
        return *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + elem);
    }
}

// 16 bytes per lane global -> LDS (buffer_load_dwordx4 ... lds): lane l's
// bytes come from `rsrc` base + `voff` and land at byte 16 l of the 1 KB at
// `lds`.  The buffer form takes the wave-uniform base from SGPRs and the lane
// offset as one 32-bit VGPR, so a DMA costs no VALU address arithmetic.  Kept
// out of the templates below: the host pass of hipcc rejects LDS-DMA builtins
// in a template body instantiated from more than one kernel.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, char* lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (LDS_AS void*)lds, 16, voff, 0, 0, 0);
}

// Raw buffer descriptor over `p` (bytes from p on are addressable; every
// offset the kernel forms stays inside the tensor).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const char* p) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p), (short)0, 0x7fffffff, 0x00020000);
}

// A wave-uniform pointer, moved to scalar registers.
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<const char*>(((uint64_t)hi << 32) | lo);
}

// Per-lane constants of the tile DMA: LDS DMA (global_load_lds_dwordx4)
// writes lane l's 16 bytes at byte 16 l of the wave's 1 KB chunk, so each lane
// fetches the global 16 bytes that belong at that swizzled LDS position: unit
// p = 64 * chunk + l of the tile is row p / UPR, physical unit p % UPR.
template <int D, bool IS_V, int NW>
struct DmaLane {
    uint32_t off[Cfg<D, NW>::CPW];  // byte offset of the lane's 16 bytes within the tile's global rows
    int row[Cfg<D, NW>::CPW];       // tile row of those bytes
    __device__ __forceinline__ void init(int wave, int lane) {
        using C = Cfg<D, NW>;
#pragma unroll
        for (int i = 0; i < C::CPW; ++i) {
            const int p = (wave * C::CPW + i) * 64 + lane;
            const int r = p / C::UPR, phys = p % C::UPR;
            const int u = IS_V ? v_unit<D>(r, phys) : k_unit<D>(r, phys);
            row[i] = r;
            off[i] = (uint32_t)(r * C::RB + u * 16);
        }
    }
};

// Stage one K or V tile (keys t0 .. t0+63 of a block of n keys) into the LDS
// region at byte `lds_off`.  bf16 sources go global -> LDS directly; rows past
// the block end are clamped to its last row (finite data whose scores are
// masked to -inf and whose softmax weights are 0).  fp16 sources take the bf16
// path (16-bit elements either way).  fp32 sources are read into registers,
// rounded to bf16 and stored.  `wave` must be wave-uniform (it
// selects the LDS chunk, which the DMA takes from M0).
template <bool F32, int D, bool IS_V, int NW>
__device__ __forceinline__ void stage_tile(char* smem, int lds_off, const char* src, int t0, int n,
                                           const DmaLane<D, IS_V, NW>& dl, int wave, int lane) {
    using C = Cfg<D, NW>;
    const char* tile = uniform_ptr(src + (size_t)t0 * (F32 ? 2 * C::RB : C::RB));
    char* dst0 = smem + lds_off + wave * C::CPW * 1024;
    if (t0 + BN <= n) {
#pragma unroll
        for (int i = 0; i < C::CPW; ++i) {
            if constexpr (F32) {
                *reinterpret_cast<u32x4*>(dst0 + i * 1024 + lane * 16) = load8<true>(tile, dl.off[i] / 2);
            } else {
                dma16(raw_rsrc(tile), dl.off[i], dst0 + i * 1024);
            }
        }
    } else {
        const int last = n - 1 - t0;
#pragma unroll
        for (int i = 0; i < C::CPW; ++i) {
            const uint32_t off = dl.off[i] - (uint32_t)((dl.row[i] - min(dl.row[i], last)) * C::RB);
            if constexpr (F32) {
                *reinterpret_cast<u32x4*>(dst0 + i * 1024 + lane * 16) = load8<true>(tile, off / 2);
            } else {
                dma16(raw_rsrc(tile), off, dst0 + i * 1024);
            }
        }
    }
}

// Row max of a 64-key tile (both lane halves), in log2 units.
__device__ __forceinline__ float tile_max(const f32x16 (&s)[2], float sl2) {
    float m[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) m[j] = fmaxf(s[0][j], s[1][j]);
#pragma unroll
    for (int i = 4; i < 16; i += 4)
#pragma unroll
        for (int j = 0; j < 4; ++j) m[j] = fmaxf(m[j], fmaxf(s[0][i + j], s[1][i + j]));
    return pair_max(fmaxf(fmaxf(m[0], m[1]), fmaxf(m[2], m[3]))) * sl2;
}

template <int D, int IN, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2)))
void attn_fwd_kernel(AttnArgs a) {
    using C = Cfg<D, NW>;
    constexpr int BM = C::BM;
    constexpr bool F32 = IN == DT_F32;
    typedef typename Op<IN>::T8 op8;
    __shared__ __attribute__((aligned(1024))) char smem[C::LDS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int h = lane >> 5;    // lane half
    const int c32 = lane & 31;  // query column within the wave's 32

    // XCD-aware mapping of workgroup id -> (plane, query tile).
    const int nblk = gridDim.x;
    const int bid = blockIdx.x;
    const int per = nblk >> 3, rem = nblk & 7;
    const int xcd = bid & 7, idx = bid >> 3;
    const int logical = xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
    const int nq = (int)((a.Sq + BM - 1) / BM);
    const int64_t plane = logical / nq;
    const int qt = logical - (int)plane * nq;

    const int64_t Sq = a.Sq;
    const int n = (int)a.Skv;
    const int64_t qrow = (int64_t)qt * BM + wave * 32 + c32;
    const bool qvalid = qrow < Sq;

    const size_t esz = F32 ? 4 : 2;
    const char* qp = static_cast<const char*>(a.q) + (size_t)(plane * Sq) * D * esz;
    const char* kp = static_cast<const char*>(a.k) + (size_t)(plane * a.kv_plane) * esz;
    const char* vp = static_cast<const char*>(a.v) + (size_t)(plane * a.kv_plane) * esz;

    // Q^T fragments: lane holds q[qrow][16*kk + 8*h .. +7] (rows past Sq read row Sq-1, then zeroed).
    op8 qf[C::NK];
    {
        const int64_t qr = qvalid ? qrow : Sq - 1;
#pragma unroll
        for (int kk = 0; kk < C::NK; ++kk) {
            u32x4 x = load8<F32>(qp, qr * D + kk * 16 + h * 8);
            if (!qvalid) x = u32x4{0, 0, 0, 0};
            qf[kk] = __builtin_bit_cast(op8, x);
        }
    }

    f32x16 o[C::NDB];
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] = 0.f;

    float m_run = -INFINITY;  // exponent base (log2 units), identical in lanes l and l^32
    float l_run = 0.f;        // this lane's share of the row sum
    const float sl2 = a.scale_log2;

    // Per-lane LDS read offsets (tile-relative); stage and (kb, ks, r) parts are immediates.
    // K fragment (S^T A operand): key row kb*32 + c32, d-units 2*kk + h; the
    // swizzle depends on the row only through c32.
    int k_lane[C::NK];
#pragma unroll
    for (int kk = 0; kk < C::NK; ++kk) k_lane[kk] = c32 * C::RB + k_unit<D>(c32, 2 * kk + h) * 16;
    // V^T fragment (O^T A operand) via ds_read_b64_tr_b16: in each 16-lane
    // group, lane m = 4a + b reads the 4 values [d0 + 4b, +4) of key row
    // 16*ks + 8r + 4h + a; the transposed result gives lane i the values at
    // d0 + i of those 4 keys -- k-slots 8h + 4r .. +3 of the MFMA, which the
    // S^T accumulator layout assigns to exactly those keys.  The swizzle
    // depends on the row only through 4h + a.
    int v_lane[C::NDB];
    {
        const int tr_g = lane >> 4, tr_m = lane & 15, tr_a = tr_m >> 2, tr_b = tr_m & 3;
        const int row = 4 * h + tr_a;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
            const int d0 = 32 * db + 16 * (tr_g & 1) + 4 * tr_b;
            v_lane[db] = row * C::RB + v_unit<D>(row, d0 >> 3) * 16 + (d0 & 7) * 2;
        }
    }
    DmaLane<D, false, NW> kdl;
    DmaLane<D, true, NW> vdl;
    kdl.init(wave, lane);
    vdl.init(wave, lane);

    const int ntiles = (n + BN - 1) / BN;
    if (ntiles > 0) {
        stage_tile<F32>(smem, 0, kp, 0, n, kdl, wave, lane);
        stage_tile<F32>(smem, 2 * C::TILE, vp, 0, n, vdl, wave, lane);
    }

    // One tile: wait for its DMA, start the next tile's DMA into the other
    // stage, S^T = K Q^T, softmax, O^T += V^T P^T.  STG (the stage holding the
    // tile) is a compile-time constant, so every LDS address is a per-lane
    // base plus an immediate.
    auto step = [&](auto stg_c, int t) __attribute__((always_inline)) {
        constexpr int STG = decltype(stg_c)::value;
        constexpr int K_CUR = STG * C::TILE, V_CUR = (2 + STG) * C::TILE;
        constexpr int K_NXT = (1 - STG) * C::TILE, V_NXT = (3 - STG) * C::TILE;
        // tile t has landed for every wave; every wave is done with the other stage
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (t + 1 < ntiles) {
            stage_tile<F32>(smem, K_NXT, kp, (t + 1) * BN, n, kdl, wave, lane);
            stage_tile<F32>(smem, V_NXT, vp, (t + 1) * BN, n, vdl, wave, lane);
        }

        // S^T (64 keys x 32 queries) = K_tile . Q^T
        f32x16 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
#pragma unroll
        for (int kk = 0; kk < C::NK; ++kk)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const op8 kf = *reinterpret_cast<const op8*>(smem + K_CUR + kb * 32 * C::RB + k_lane[kk]);
                s[kb] = mfma32x32x16(kf, qf[kk], s[kb]);
            }
        // keep four K-fragment reads in flight ahead of the MFMAs that consume them
#pragma unroll
        for (int i = 0; i < 4; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
#pragma unroll
        for (int i = 0; i < 12; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);

        // Keys past the end of the block never enter the softmax.
        const int t0 = t * BN;
        if (t0 + BN > n) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = t0 + kb * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
                    if (key >= n) s[kb][i] = -INFINITY;
                }
        }

        const float mt = tile_max(s, sl2);
        const bool need = mt > m_run + kSlack;
        float alpha = 1.f;
        if (need) {
            alpha = exp2_fast(m_run - mt);
            m_run = mt;
        }
        const float neg_m = -m_run;
        float rs0 = 0.f, rs1 = 0.f;
        op8 pb[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int kb = ks >> 1, base = (ks & 1) * 8;
            f32x8 p;
#pragma unroll
            for (int j = 0; j < 8; ++j) p[j] = exp2_fast(fmaf(s[kb][base + j], sl2, neg_m));
            pb[ks] = __builtin_convertvector(p, op8);
#pragma unroll
            for (int j = 0; j < 8; j += 2) {
                rs0 += p[j];
                rs1 += p[j + 1];
            }
        }
        l_run = l_run * alpha + (rs0 + rs1);
        if (__any(need)) {
#pragma unroll
            for (int db = 0; db < C::NDB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
        }

        // O^T += V^T . P^T, 16 keys per MFMA.
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
            for (int db = 0; db < C::NDB; ++db) {
                const char* vb = smem + V_CUR + 16 * ks * C::RB + v_lane[db];
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(vb));
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(vb + 8 * C::RB));
                const s16x4 lohi[2] = {lo, hi};
                const op8 vf = __builtin_bit_cast(op8, lohi);
                o[db] = mfma32x32x16(vf, pb[ks], o[db]);
            }
        }
    };

    for (int t = 0; t < ntiles; t += 2) {
        step(std::integral_constant<int, 0>(), t);
        if (t + 1 < ntiles) step(std::integral_constant<int, 1>(), t + 1);
    }

    // Epilogue: normalise, then store or LSE-merge into the accumulator.
    const float l_tot = pair_sum(l_run);
    const bool any_key = l_tot > 0.f;
    const float inv_l = any_key ? 1.f / l_tot : 0.f;
    const float lse2 = any_key ? m_run + log2_fast(l_tot) : -INFINITY;  // log2 units
    if (!qvalid) return;

    float wa = 0.f, wb = inv_l, lnew2 = lse2;
    const char* acc = nullptr;
    bool acc_empty = true;  // accumulator LSE -inf (bit test: its values are never read then)
    if (a.mode == EPI_MERGE) {
        const float la_raw = a.lse_in[plane * Sq + qrow];
        acc_empty = __float_as_uint(la_raw) == 0xff800000u;
        const float la2 = la_raw * kLog2e;
        const float mx = fmaxf(la2, lse2);
        if (mx == -INFINITY) {
            wa = 0.f;
            wb = 0.f;
            lnew2 = -INFINITY;
        } else {
            const float ea = exp2_fast(la2 - mx);
            const float eb = exp2_fast(lse2 - mx);
            const float tot = ea + eb;
            const float it = 1.f / tot;
            wa = ea * it;
            wb = eb * it * inv_l;
            lnew2 = mx + log2_fast(tot);
        }
        acc = static_cast<const char*>(a.acc_in) + (size_t)(plane * Sq + qrow) * D * (a.acc_dtype == DT_F32 ? 4 : 2);
    }

    const size_t orow = (size_t)(plane * Sq + qrow) * D;
    // lane owns d-values db*32 + g4*8 + h*4 .. +3 of its query row
    f32x4 r[C::NDB * 4];
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            f32x4 x = {o[db][g4 * 4 + 0] * wb, o[db][g4 * 4 + 1] * wb, o[db][g4 * 4 + 2] * wb,
                       o[db][g4 * 4 + 3] * wb};
            if (acc != nullptr && !acc_empty) {
                const int e0 = db * 32 + g4 * 8 + h * 4;
                f32x4 av;
                if (a.acc_dtype == DT_F32)
                    av = *reinterpret_cast<const f32x4*>(acc + e0 * 4);
                else if (a.acc_dtype == DT_F16)
                    av = __builtin_convertvector(*reinterpret_cast<const f16x4*>(acc + e0 * 2), f32x4);
                else
                    av = __builtin_convertvector(*reinterpret_cast<const bf16x4*>(acc + e0 * 2), f32x4);
                x = x + av * wa;
            }
            r[db * 4 + g4] = x;
        }
    if (a.out_dtype == DT_F32) {
        float* dst = static_cast<float*>(a.out) + orow + h * 4;
#pragma unroll
        for (int i = 0; i < C::NDB * 4; ++i) *reinterpret_cast<f32x4*>(dst + i * 8) = r[i];
    } else if (a.out_dtype == DT_F16) {
        _Float16* dst = static_cast<_Float16*>(a.out) + orow + h * 4;
#pragma unroll
        for (int i = 0; i < C::NDB * 4; ++i)
            *reinterpret_cast<f16x4*>(dst + i * 8) = __builtin_convertvector(r[i], f16x4);
    } else {
        __bf16* dst = static_cast<__bf16*>(a.out) + orow + h * 4;
#pragma unroll
        for (int i = 0; i < C::NDB * 4; ++i)
            *reinterpret_cast<bf16x4*>(dst + i * 8) = __builtin_convertvector(r[i], bf16x4);
    }
    if (h == 0) a.lse_out[plane * Sq + qrow] = lnew2 * kLn2;
}

template <int D, int IN, int NW>
hipError_t launch_nw(const AttnArgs& a, hipStream_t stream) {
    using C = Cfg<D, NW>;
    const int64_t nblk = (a.Sq + C::BM - 1) / C::BM * a.n_planes;
    hipLaunchKernelGGL((attn_fwd_kernel<D, IN, NW>), dim3((unsigned)nblk), dim3(C::NT), 0, stream, a);
    return hipGetLastError();
}

// Four-wave workgroups (two resident per CU) in general; when even those fit
// the 256-CU chip in one round (512 slots), eight-wave workgroups (one per CU,
// each K/V tile staged once for 256 queries) run the same per-row arithmetic
// with half the tile traffic and half the workgroups' fixed costs.
constexpr int64_t kOneRoundSlots = 512;

template <int D, int IN>
hipError_t launch_t(const AttnArgs& a, hipStream_t stream) {
    if ((a.Sq + Cfg<D, 4>::BM - 1) / Cfg<D, 4>::BM * a.n_planes <= kOneRoundSlots)
        return launch_nw<D, IN, 8>(a, stream);
    return launch_nw<D, IN, 4>(a, stream);
}

template <int D>
hipError_t launch_d(const AttnArgs& a, hipStream_t stream) {
    switch (a.in_dtype) {
        case DT_BF16: return launch_t<D, DT_BF16>(a, stream);
        case DT_F32: return launch_t<D, DT_F32>(a, stream);
        case DT_F16: return launch_t<D, DT_F16>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_attn_fwd(const AttnArgs& a, hipStream_t stream) {
    if (a.Sq <= 0 || a.n_planes <= 0) return hipSuccess;
    if (a.out_dtype != DT_BF16 && a.out_dtype != DT_F32 && a.out_dtype != DT_F16) return hipErrorInvalidValue;
    if (a.d == 128) return launch_d<128>(a, stream);
    if (a.d == 64) return launch_d<64>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace cpattn
