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
    // byte offset of the lane's 16 bytes within the tile's global rows (its
    // tile row is off / RB: the unit part is below one row)
    uint32_t off[Cfg<D, NW>::CPW];
    __device__ __forceinline__ void init(int wave, int lane) {
        using C = Cfg<D, NW>;
#pragma unroll
        for (int i = 0; i < C::CPW; ++i) {
            const int p = (wave * C::CPW + i) * 64 + lane;
            const int r = p / C::UPR, phys = p % C::UPR;
            const int u = IS_V ? v_unit<D>(r, phys) : k_unit<D>(r, phys);
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
            const int row = (int)(dl.off[i] / C::RB);
            const uint32_t off = dl.off[i] - (uint32_t)((row - min(row, last)) * C::RB);
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


// Per-lane constants of one wave's tile work: LDS read offsets of its K and
// V^T fragments and its share of the tile DMA.
template <int D, int NW>
struct Lanes {
    using C = Cfg<D, NW>;
    int wave, lane, h, c32;
    int k_lane[C::NK];
    int v_lane[C::NDB];
    DmaLane<D, false, NW> kdl;
    DmaLane<D, true, NW> vdl;

    __device__ __forceinline__ void init(int tid) {
        lane = tid & 63;
        wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
        h = lane >> 5;    // lane half
        c32 = lane & 31;  // query column within the wave's 32
        // K fragment (S^T A operand): key row kb*32 + c32, d-units 2*kk + h; the
        // swizzle depends on the row only through c32.
#pragma unroll
        for (int kk = 0; kk < C::NK; ++kk) k_lane[kk] = c32 * C::RB + k_unit<D>(c32, 2 * kk + h) * 16;
        // V^T fragment (O^T A operand) via ds_read_b64_tr_b16: in each 16-lane
        // group, lane m = 4a + b reads the 4 values [d0 + 4b, +4) of key row
        // 16*ks + 8r + 4h + a; the transposed result gives lane i the values at
        // d0 + i of those 4 keys -- k-slots 8h + 4r .. +3 of the MFMA, which the
        // S^T accumulator layout assigns to exactly those keys.  The swizzle
        // depends on the row only through 4h + a.
        const int tr_g = lane >> 4, tr_m = lane & 15, tr_a = tr_m >> 2, tr_b = tr_m & 3;
        const int row = 4 * h + tr_a;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
            const int d0 = 32 * db + 16 * (tr_g & 1) + 4 * tr_b;
            v_lane[db] = row * C::RB + v_unit<D>(row, d0 >> 3) * 16 + (d0 & 7) * 2;
        }
        kdl.init(wave, lane);
        vdl.init(wave, lane);
    }

    // Stage keys t0 .. t0+63 of a K/V block of n keys (plane bases kp, vp)
    // into the LDS stage at K_OFF / V_OFF.
    template <bool F32>
    __device__ __forceinline__ void stage(char* smem, int k_off, int v_off, const char* kp, const char* vp, int t0,
                                          int n) const {
        stage_tile<F32>(smem, k_off, kp, t0, n, kdl, wave, lane);
        stage_tile<F32>(smem, v_off, vp, t0, n, vdl, wave, lane);
    }
};

// Running softmax state of one wave's 32 queries over the keys seen so far:
// O^T unnormalised against the exponent base m (log2 units, identical in lanes
// l and l^32) and this lane's share l of the row sum.
template <int D>
struct Run {
    f32x16 o[D / 32];
    float m, l;
    __device__ __forceinline__ void reset() {
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
        m = -INFINITY;
        l = 0.f;
    }
};

// Q^T fragments of the wave's 32 query rows: lane holds q[qrow][16*kk + 8*h .. +7]
// (rows past Sq read row Sq-1, then zeroed).
template <int D, int IN>
__device__ __forceinline__ void load_q(typename Op<IN>::T8 (&qf)[D / 16], const char* qp, int64_t qrow, int64_t Sq,
                                       int h) {
    constexpr bool F32 = IN == DT_F32;
    typedef typename Op<IN>::T8 op8;
    const bool qvalid = qrow < Sq;
    const int64_t qr = qvalid ? qrow : Sq - 1;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
        u32x4 x = load8<F32>(qp, qr * D + kk * 16 + h * 8);
        if (!qvalid) x = u32x4{0, 0, 0, 0};
        qf[kk] = __builtin_bit_cast(op8, x);
    }
}

// One 64-key tile resident in LDS stage STG: S^T = K Q^T, the online softmax
// update, O^T += V^T P^T.  The tile holds keys t0 .. t0+63 of a block of n
// keys; keys past n never enter the softmax.  Every LDS address is a
// per-lane base plus a compile-time immediate.
template <int STG, int D, int IN, int NW>
__device__ __forceinline__ void tile_math(const char* smem, const Lanes<D, NW>& ln,
                                          const typename Op<IN>::T8 (&qf)[D / 16], Run<D>& st, float sl2,
                                          int t0, int n) {
    using C = Cfg<D, NW>;
    typedef typename Op<IN>::T8 op8;
    constexpr int K_CUR = STG * C::TILE, V_CUR = (2 + STG) * C::TILE;
    const int h = ln.h;

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
            const op8 kf = *reinterpret_cast<const op8*>(smem + K_CUR + kb * 32 * C::RB + ln.k_lane[kk]);
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
    // (written against t0 and n: the form the compiler keeps out of the registers)
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
    const bool need = mt > st.m + kSlack;
    float alpha = 1.f;
    if (need) {
        alpha = exp2_fast(st.m - mt);
        st.m = mt;
    }
    const float neg_m = -st.m;
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
    st.l = st.l * alpha + (rs0 + rs1);
    if (__any(need)) {
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) st.o[db][i] *= alpha;
    }

    // O^T += V^T . P^T, 16 keys per MFMA.
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
            const char* vb = smem + V_CUR + 16 * ks * C::RB + ln.v_lane[db];
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(vb));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(vb + 8 * C::RB));
            const s16x4 lohi[2] = {lo, hi};
            const op8 vf = __builtin_bit_cast(op8, lohi);
            st.o[db] = mfma32x32x16(vf, pb[ks], st.o[db]);
        }
    }
}

// XCD-aware order: workgroups go round-robin over the 8 XCDs, so each XCD is
// given a contiguous range of logical ids (and with it of planes, whose K/V then
// stays in that XCD's L2).
__device__ __forceinline__ int xcd_logical(int bid, int nblk) {
    const int per = nblk >> 3, rem = nblk & 7;
    const int xcd = bid & 7, idx = bid >> 3;
    return xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
}

// Store 4 consecutive output values of element type `dt` at `dst` (element offset e).
__device__ __forceinline__ void store4(void* dst, size_t e, int dt, f32x4 x) {
    if (dt == DT_F32)
        *reinterpret_cast<f32x4*>(static_cast<float*>(dst) + e) = x;
    else if (dt == DT_F16)
        *reinterpret_cast<f16x4*>(static_cast<_Float16*>(dst) + e) = __builtin_convertvector(x, f16x4);
    else
        *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(dst) + e) = __builtin_convertvector(x, bf16x4);
}

template <int D, int IN, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2)))
void attn_fwd_kernel(AttnArgs a) {
    using C = Cfg<D, NW>;
    constexpr int BM = C::BM;
    constexpr bool F32 = IN == DT_F32;
    typedef typename Op<IN>::T8 op8;
    __shared__ __attribute__((aligned(1024))) char smem[C::LDS];

    Lanes<D, NW> ln;
    ln.init(threadIdx.x);
    const int h = ln.h;

    const int logical = xcd_logical(blockIdx.x, gridDim.x);
    const int nq = (int)((a.Sq + BM - 1) / BM);
    const int64_t plane = logical / nq;
    const int qt = logical - (int)plane * nq;

    const int64_t Sq = a.Sq;
    const int n = (int)a.Skv;
    const int64_t qrow = (int64_t)qt * BM + ln.wave * 32 + ln.c32;
    const bool qvalid = qrow < Sq;

    const size_t esz = F32 ? 4 : 2;
    const char* qp = static_cast<const char*>(a.q) + (size_t)(plane * Sq) * D * esz;
    const char* kp = static_cast<const char*>(a.k) + (size_t)(plane * a.kv_plane) * esz;
    const char* vp = static_cast<const char*>(a.v) + (size_t)(plane * a.kv_plane) * esz;

    op8 qf[C::NK];
    load_q<D, IN>(qf, qp, qrow, Sq, h);
    Run<D> st;
    st.reset();
    const float sl2 = a.scale_log2;

    const int ntiles = (n + BN - 1) / BN;
    if (ntiles > 0) ln.template stage<F32>(smem, 0, 2 * C::TILE, kp, vp, 0, n);

    // One tile: wait for its DMA, start the next tile's DMA into the other
    // stage, then the math.  STG (the stage holding the tile) is a compile-time
    // constant.
    auto step = [&](auto stg_c, int t) __attribute__((always_inline)) {
        constexpr int STG = decltype(stg_c)::value;
        // tile t has landed for every wave; every wave is done with the other stage
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (t + 1 < ntiles)
            ln.template stage<F32>(smem, (1 - STG) * C::TILE, (3 - STG) * C::TILE, kp, vp, (t + 1) * BN, n);
        tile_math<STG, D, IN, NW>(smem, ln, qf, st, sl2, t * BN, n);
    };

    for (int t = 0; t < ntiles; t += 2) {
        step(std::integral_constant<int, 0>(), t);
        if (t + 1 < ntiles) step(std::integral_constant<int, 1>(), t + 1);
    }

    // Epilogue: normalise, then store or LSE-merge into the accumulator.
    const float l_tot = pair_sum(st.l);
    const bool any_key = l_tot > 0.f;
    const float inv_l = any_key ? 1.f / l_tot : 0.f;
    const float lse2 = any_key ? st.m + log2_fast(l_tot) : -INFINITY;  // log2 units
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
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const int e0 = db * 32 + g4 * 8 + h * 4;
            f32x4 x = {st.o[db][g4 * 4 + 0] * wb, st.o[db][g4 * 4 + 1] * wb, st.o[db][g4 * 4 + 2] * wb,
                       st.o[db][g4 * 4 + 3] * wb};
            if (acc != nullptr && !acc_empty) {
                f32x4 av;
                if (a.acc_dtype == DT_F32)
                    av = *reinterpret_cast<const f32x4*>(acc + e0 * 4);
                else if (a.acc_dtype == DT_F16)
                    av = __builtin_convertvector(*reinterpret_cast<const f16x4*>(acc + e0 * 2), f32x4);
                else
                    av = __builtin_convertvector(*reinterpret_cast<const bf16x4*>(acc + e0 * 2), f32x4);
                x = x + av * wa;
            }
            store4(a.out, orow + e0, a.out_dtype, x);
        }
    if (h == 0) a.lse_out[plane * Sq + qrow] = lnew2 * kLn2;
}

// ---------------------------------------------------------------------------
// Ring step in one launch.
//
// The work of a ring step is, for every (plane, query tile), the key tiles of
// chunk 0, then chunk 1, ... in ring order: T tiles (each chunk tiled on its
// own, so a tile never straddles two chunks).  The launch's S workgroups (S =
// the chip's resident slots) take it in rounds:
//   * R = Q / S full rounds over the Q query tiles: workgroup w runs query tile
//     r*S + w whole in round r.  Every workgroup starts a round at key tile 0
//     and all move through the keys at the same pace, so the workgroups of an
//     XCD (consecutive query tiles of the same planes) read the same K/V tiles
//     at the same time and the XCD's L2 serves them.
//   * The L = Q % S query tiles left over are balanced over all S workgroups:
//     each is cut at key tile a = round(L*T/S) into a head [0, a), run by
//     workgroup i < L (again all in step), and a tail [a, T); the L tails, laid
//     end to end, are split into S - L equal contiguous ranges, one per
//     remaining workgroup.  Every workgroup then holds about L*T/S tiles.
// Within a piece the online softmax runs tile by tile; at the end of every
// chunk the running state is closed: output normalised and LSE formed in fp32
// -- the ring's merged accumulator after that chunk -- and the next chunk
// continues from it (close_chunk).  A query tile run whole is written out; the
// pieces of a cut one (fp32 output and LSE) go to the workspace and
// ring_fixup_kernel merges them in key order by the log-sum-exp identity.  No
// atomics: the result is bitwise repeatable.
//
// Workspace slots (slot_rows x D fp32 outputs, slot_rows LSEs each): head of
// leftover tile i -> slot i; the first / last piece of tail range t (when it
// cuts a tail) -> L + 2t / L + 2t + 1; a tail run whole inside one range ->
// L + 2(S - L) + i.  At most 2S slots.
// ---------------------------------------------------------------------------

// First unit of range w when n units are split into ranges of per = n / k units,
// the first rem = n % k of them one longer.
__device__ __forceinline__ int64_t range_begin(int64_t w, int64_t per, int64_t rem) {
    return w * per + (w < rem ? w : rem);
}
// The range holding unit x (inverse of range_begin).
__device__ __forceinline__ int64_t range_of(int64_t x, int64_t per, int64_t rem) {
    const int64_t big = rem * (per + 1);
    return x < big ? x / (per + 1) : rem + (x - big) / per;
}

// Close a chunk: the running state becomes the fp32 accumulator of every
// chunk seen so far -- output normalised (o / l) and its LSE m + log2 l formed --
// and is handed to the next chunk as its starting state: base m = that LSE,
// weight 1 (half in each lane half).  The next chunk's tiles then fold into it
// by the online rescale, which is the log-sum-exp merge of the accumulator with
// that chunk's partial: at its close, o / l = (acc * a + sum_j p_j v_j) / (a + sum_j p_j)
// with a = exp2(LSE_acc - base), i.e. the merge weights of the two LSEs.
template <int D>
__device__ __forceinline__ void close_chunk(Run<D>& st) {
    const float l_tot = pair_sum(st.l);  // >= 1: the tile that set the base holds a weight of 1
    const float inv_l = 1.f / l_tot;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) st.o[db][i] *= inv_l;
    st.m = st.m + log2_fast(l_tot);
    st.l = 0.5f;
}

// One piece: key tiles [g0, g1) of query tile qi, then its store -- whole
// (g0 == 0 and g1 == T) to the output, else to workspace slot `slot`.
template <int D, int IN, int NW>
__device__ __forceinline__ void ring_piece(const RingArgs& a, char* smem, const Lanes<D, NW>& ln, int64_t qi, int g0,
                                           int g1, int64_t slot) {
    using C = Cfg<D, NW>;
    constexpr int BM = C::BM;
    constexpr bool F32 = IN == DT_F32;
    typedef typename Op<IN>::T8 op8;
    const int h = ln.h;
    const int T = a.T;
    const int64_t Sq = a.Sq;
    const size_t esz = F32 ? 4 : 2;
    const int64_t plane = qi / a.nq;
    const int qt = (int)(qi - plane * a.nq);
    const int rloc = ln.wave * 32 + ln.c32;  // query row within the tile
    const int64_t qrow = (int64_t)qt * BM + rloc;

    const char* qp = static_cast<const char*>(a.q) + (size_t)(plane * Sq) * D * esz;
    const char* kp = static_cast<const char*>(a.k) + (size_t)(plane * a.kv_plane) * esz;
    const char* vp = static_cast<const char*>(a.v) + (size_t)(plane * a.kv_plane) * esz;
    op8 qf[C::NK];
    load_q<D, IN>(qf, qp, qrow, Sq, h);

    // chunk and chunk-local tile of unit g0 (the table holds only non-empty chunks)
    int c = 0;
    while (a.chunk_tile0[c + 1] <= g0) ++c;
    int t = g0 - a.chunk_tile0[c];
    int len = a.chunk_len[c];
    // the tile after the current one (its chunk's offset and length), known a step ahead so
    // that the DMA issued after each barrier needs no table load
    int nc = c, nt = t + 1, noff = a.chunk_off[c], nlen = len;
    if (nt * BN >= len) {
        nc = c + 1 < a.n_chunks ? c + 1 : c;
        nt = 0;
        noff = a.chunk_off[nc];
        nlen = a.chunk_len[nc];
    }

    Run<D> st;
    st.reset();
    const float sl2 = a.scale_log2;

    // every wave is done reading the stages of the previous piece
    __syncthreads();
    {
        const size_t co = (size_t)a.chunk_off[c] * D * esz;
        ln.template stage<F32>(smem, 0, 2 * C::TILE, kp + co, vp + co, t * BN, len);
    }

    auto step = [&](auto stg_c, int g) __attribute__((always_inline)) {
        constexpr int STG = decltype(stg_c)::value;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (g + 1 < g1) {
            const size_t co = (size_t)noff * D * esz;
            ln.template stage<F32>(smem, (1 - STG) * C::TILE, (3 - STG) * C::TILE, kp + co, vp + co, nt * BN, nlen);
        }
        const bool chunk_end = (t + 1) * BN >= len;
        tile_math<STG, D, IN, NW>(smem, ln, qf, st, sl2, t * BN, len);
        if (chunk_end || g + 1 == g1) close_chunk<D>(st);
        // advance: current <- next, next <- the tile after it
        c = nc;
        t = nt;
        len = nlen;
        ++nt;
        if (nt * BN >= nlen) {
            nc = nc + 1 < a.n_chunks ? nc + 1 : nc;
            nt = 0;
            noff = a.chunk_off[nc];
            nlen = a.chunk_len[nc];
        }
    };
    for (int g = g0; g < g1; g += 2) {
        step(std::integral_constant<int, 0>(), g);
        if (g + 1 < g1) step(std::integral_constant<int, 1>(), g + 1);
    }

    if (qrow < Sq) {
        if (g0 == 0 && g1 == T) {
            const size_t orow = (size_t)(plane * Sq + qrow) * D;
#pragma unroll
            for (int db = 0; db < C::NDB; ++db)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const f32x4 x = {st.o[db][g4 * 4 + 0], st.o[db][g4 * 4 + 1], st.o[db][g4 * 4 + 2],
                                     st.o[db][g4 * 4 + 3]};
                    store4(a.out, orow + db * 32 + g4 * 8 + h * 4, a.out_dtype, x);
                }
            if (h == 0) a.lse_out[plane * Sq + qrow] = st.m * kLn2;
        } else {
            float* po = a.part_o + (size_t)(slot * a.slot_rows + rloc) * D;
#pragma unroll
            for (int db = 0; db < C::NDB; ++db)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const f32x4 x = {st.o[db][g4 * 4 + 0], st.o[db][g4 * 4 + 1], st.o[db][g4 * 4 + 2],
                                     st.o[db][g4 * 4 + 3]};
                    *reinterpret_cast<f32x4*>(po + db * 32 + g4 * 8 + h * 4) = x;
                }
            if (h == 0) a.part_lse[slot * a.slot_rows + rloc] = st.m;  // log2 units
        }
    }
}

template <int D, int IN, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(kRingWavesPerSimd<D>)))
void attn_ring_kernel(RingArgs a) {
    using C = Cfg<D, NW>;
    __shared__ __attribute__((aligned(1024))) char smem[C::LDS];

    Lanes<D, NW> ln;
    ln.init(threadIdx.x);
    const int S = gridDim.x;
    const int w = xcd_logical(blockIdx.x, S);
    const int T = a.T;

    // The workgroup's pieces in order -- its whole tiles of the full rounds, then
    // its head or its tail range -- through one call site (one inlined copy).
    const int R = a.rounds, L = a.left, H = a.head, TT = T - H;
    const int64_t q0 = (int64_t)R * S;  // first leftover query tile
    const int64_t tw = w - L;           // tail range of this workgroup (if w >= L)
    int64_t u = 0, u_end = 0;           // its tail units
    if (L > 0 && w >= L) {
        u = range_begin(tw, a.tail_per, a.tail_rem);
        u_end = range_begin(tw + 1, a.tail_per, a.tail_rem);
    }
    const int64_t u_first = u;
    bool head = L > 0 && w < L && H > 0;
    for (int r = 0;;) {
        int64_t qi, slot = 0;
        int g0, g1;
        if (r < R) {
            qi = (int64_t)r * S + w;
            g0 = 0;
            g1 = T;
            ++r;
        } else if (head) {
            qi = q0 + w;
            g0 = 0;
            g1 = H;
            slot = w;
            head = false;
        } else if (u < u_end) {
            const int64_t i = u / TT;
            const int t0 = (int)(u - i * TT);
            const int t1 = (int)min((int64_t)TT, (int64_t)t0 + (u_end - u));
            qi = q0 + i;
            g0 = H + t0;
            g1 = H + t1;
            slot = (t0 == 0 && t1 == TT) ? L + 2 * (int64_t)(S - L) + i : L + 2 * tw + (u == u_first ? 0 : 1);
            u += t1 - t0;
        } else {
            break;
        }
        ring_piece<D, IN, NW>(a, smem, ln, qi, g0, g1, slot);
    }
}

// Merge the pieces of leftover query tile i (blockIdx.y), in key order, into the
// output: one thread per 4 output values (blockIdx.x picks 256 of the tile's
// rows x D/4).  Tiles run whole (a head of all T tiles, or, with no heads, a
// tail inside one range) were written out by their workgroup.
template <int D>
__global__ __launch_bounds__(256) void ring_fixup_kernel(RingArgs a, int BM) {
    const int64_t i = blockIdx.y;
    const int L = a.left, H = a.head, T = a.T, S = a.n_ranges;
    const int TT = T - H;
    if (TT == 0) return;                      // heads were whole tiles
    const int64_t ts = i * TT, te = ts + TT;  // the tail's units
    const int64_t w0 = range_of(ts, a.tail_per, a.tail_rem), w1 = range_of(te - 1, a.tail_per, a.tail_rem);
    if (H == 0 && w0 == w1) return;           // a whole tile, written out
    const int64_t qi = (int64_t)a.rounds * S + i;
    const int64_t plane = qi / a.nq;
    const int qt = (int)(qi - plane * a.nq);
    constexpr int Q4 = D / 4;
    const int it = blockIdx.x * 256 + threadIdx.x;
    const int r = it / Q4, c4 = it - r * Q4;
    const int64_t qrow = (int64_t)qt * BM + r;
    if (r >= BM || qrow >= a.Sq) return;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float al = -INFINITY;
    bool first = true;
    auto fold = [&](int64_t slot) {
        const float lp = a.part_lse[slot * a.slot_rows + r];
        const f32x4 op = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4*>(a.part_o + (size_t)(slot * a.slot_rows + r) * D + c4 * 4));
        if (first) {
            acc = op;
            al = lp;
            first = false;
        } else {
            const float mx = fmaxf(al, lp);
            const float ea = exp2_fast(al - mx);
            const float eb = exp2_fast(lp - mx);
            const float tot = ea + eb;
            const float inv = 1.f / tot;
            acc = op * (eb * inv) + acc * (ea * inv);
            al = mx + log2_fast(tot);
        }
    };
    if (H > 0) fold(i);
    if (w0 == w1) {
        fold(L + 2 * (int64_t)(S - L) + i);
    } else {
        for (int64_t t = w0; t <= w1; ++t) fold(L + 2 * t + (range_begin(t, a.tail_per, a.tail_rem) < ts ? 1 : 0));
    }
    store4(a.out, (size_t)(plane * a.Sq + qrow) * D + c4 * 4, a.out_dtype, acc);
    if (c4 == 0) a.lse_out[plane * a.Sq + qrow] = al * kLn2;
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

template <int D, int IN, int NW>
hipError_t launch_ring_nw(const RingArgs& a, hipStream_t stream) {
    constexpr int BM = Cfg<D, NW>::BM;
    hipLaunchKernelGGL((attn_ring_kernel<D, IN, NW>), dim3((unsigned)a.n_ranges), dim3(64 * NW), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.left == 0 || a.head == a.T) return e;
    const unsigned per_tile = (unsigned)((BM * (D / 4) + 255) / 256);
    hipLaunchKernelGGL((ring_fixup_kernel<D>), dim3(per_tile, (unsigned)a.left), dim3(256), 0, stream, a, BM);
    return hipGetLastError();
}

template <int D, int IN>
hipError_t launch_ring_t(const RingArgs& a, hipStream_t stream) {
    // the plan picks eight waves for whole-tile steps and kRingSplitWaves for split ones
    if constexpr (kRingSplitWaves == 8) {
        return a.nw == 8 ? launch_ring_nw<D, IN, 8>(a, stream) : hipErrorInvalidValue;
    } else {
        if (a.nw == 8) return launch_ring_nw<D, IN, 8>(a, stream);
        return launch_ring_nw<D, IN, kRingSplitWaves>(a, stream);
    }
}

template <int D>
hipError_t launch_ring_d(const RingArgs& a, hipStream_t stream) {
    switch (a.in_dtype) {
        case DT_BF16: return launch_ring_t<D, DT_BF16>(a, stream);
        case DT_F32: return launch_ring_t<D, DT_F32>(a, stream);
        case DT_F16: return launch_ring_t<D, DT_F16>(a, stream);
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

hipError_t launch_attn_ring(const RingArgs& a, hipStream_t stream) {
    if (a.Sq <= 0 || a.n_planes <= 0 || a.T <= 0) return hipSuccess;
    if (a.out_dtype != DT_BF16 && a.out_dtype != DT_F32 && a.out_dtype != DT_F16) return hipErrorInvalidValue;
    if (a.d == 128) return launch_ring_d<128>(a, stream);
    if (a.d == 64) return launch_ring_d<64>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace cpattn
