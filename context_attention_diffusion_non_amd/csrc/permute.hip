// Ulysses sequence <-> head regroup: a strided-to-contiguous row copy.
//
// "Context parallelism" page, Ulysses Attention: after the all-to-all a rank
// holds the whole sequence for its share of the heads; this kernel is the local half of
// that regroup (and of its inverse), a pure copy of d-element rows:
//   seq -> head:  out[g'][b][h'][r*S_local + s][:] = in[r][b][s][g*H/P + h'][:]
//   head -> seq:  the inverse map.
// Internally the shard count P and the head-group count G may differ, and the
// seq -> head direction may rotate the shards (output block r from shard
// (r + rot) % P): Unified attention regroups the K/V shards of a whole ring x
// Ulysses grid into one head group, in the ring order of one rank.
// Each thread moves UNR units of U bytes (the largest power of two <= 16 that
// divides a row), loads first, then stores; rows of whole 16-byte units move
// one unit per thread with non-temporal loads and stores (every byte is
// touched once, and many small workgroups keep the most bytes in flight).
// Threads walk the source contiguously; a wave's stores land as whole 128-byte
// pieces of d-element rows.  Index decomposition uses multiply-high division
// by host-computed magic numbers, so the copy stays memory-bound.
// Grid: x over (b, s, h', unit) of one (rank, group) slice, y = rank r,
// z = group.  Packing q, k and v along B (as one all-to-all buffer would)
// permutes all three in one launch.
#include "internal.h"


namespace cpattn {
namespace {

constexpr int NT = 256;

typedef unsigned nt_u32x4 __attribute__((ext_vector_type(4)));

// n / d for 0 <= n < 2^31 and 1 <= d < 2^31 (round-up multiplier method):
// l = ceil(log2 d), m = floor(2^32 (2^l - d) / d) + 1, n / d = (mulhi(m, n) + n) >> l.
struct FastDiv {
    uint32_t d, m, l;
};

FastDiv make_fastdiv(uint32_t d) {
    uint32_t l = 0;
    while ((uint64_t(1) << l) < d) ++l;
    const uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1;
    return FastDiv{d, (uint32_t)m, l};
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f) {
    return (__umulhi(n, f.m) + n) >> f.l;
}

template <int U>
struct Unit;
template <> struct Unit<16> { typedef uint4 T; };
template <> struct Unit<8> { typedef uint2 T; };
template <> struct Unit<4> { typedef uint32_t T; };
template <> struct Unit<2> { typedef uint16_t T; };
template <> struct Unit<1> { typedef uint8_t T; };

struct PermGeom {
    FastDiv upr;       // units per row
    FastDiv hp;        // heads per group
    FastDiv s_loc;     // tokens per shard
    uint32_t n_units;  // units per (rank, group) slice = B * S_loc * hp * upr
    int64_t B, S_loc, H, S, hpv, uprv;
    int g0;            // first group
    int direction;
    int P;             // shards
    int rot;           // seq -> head shard rotation
};

template <int U, int UNR>
__global__ __launch_bounds__(NT) void permute_kernel(const char* __restrict__ in, char* __restrict__ out,
                                                     PermGeom g) {
    typedef typename Unit<U>::T T;
    const int64_t r = blockIdx.y;       // sequence block of the head layout
    const int64_t gi = blockIdx.z;      // group index within this call
    const int64_t grp = g.g0 + gi;
    const int64_t shard = (r + g.rot) % g.P;  // sequence shard it comes from (rot = 0 for head -> seq)
    // element-row strides, in units
    const int64_t seq_base = ((shard * g.B) * g.S_loc * g.H + grp * g.hpv) * g.uprv;  // in [P,B,S_loc,H,row]
    const int64_t head_base = (gi * g.B * g.hpv * g.S + r * g.S_loc) * g.uprv;    // in [G,B,hp,S,row]

    T val[UNR];
    int64_t dst[UNR];
    bool ok[UNR];
#pragma unroll
    for (int j = 0; j < UNR; ++j) {
        const uint32_t x = ((uint32_t)blockIdx.x * UNR + j) * NT + threadIdx.x;
        ok[j] = x < g.n_units;
        if (!ok[j]) continue;
        const uint32_t y = fdiv(x, g.upr);
        const uint32_t u = x - y * g.upr.d;
        const uint32_t z = fdiv(y, g.hp);
        const uint32_t hh = y - z * g.hp.d;
        const uint32_t b = fdiv(z, g.s_loc);
        const uint32_t s = z - b * g.s_loc.d;
        const int64_t seq_idx = seq_base + (((int64_t)b * g.S_loc + s) * g.H + hh) * g.uprv + u;
        const int64_t head_idx = head_base + (((int64_t)b * g.hpv + hh) * g.S + s) * g.uprv + u;
        const int64_t src = g.direction == 0 ? seq_idx : head_idx;
        dst[j] = g.direction == 0 ? head_idx : seq_idx;
        if constexpr (U == 16)
            val[j] = __builtin_bit_cast(T, __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4*>(in) + src));
        else
            val[j] = reinterpret_cast<const T*>(in)[src];
    }
#pragma unroll
    for (int j = 0; j < UNR; ++j) {
        if (!ok[j]) continue;
        if constexpr (U == 16)
            __builtin_nontemporal_store(__builtin_bit_cast(nt_u32x4, val[j]), reinterpret_cast<nt_u32x4*>(out) + dst[j]);
        else
            reinterpret_cast<T*>(out)[dst[j]] = val[j];
    }
}

template <int U>
hipError_t launch_u(const PermuteArgs& a, const PermGeom& g, int ngroups, hipStream_t stream) {
    constexpr int UNR = U == 16 ? 1 : 4;
    const uint32_t nblk = (uint32_t)(((int64_t)g.n_units + NT * UNR - 1) / (NT * UNR));
    hipLaunchKernelGGL((permute_kernel<U, UNR>), dim3(nblk, (unsigned)a.degree, (unsigned)ngroups), dim3(NT), 0,
                       stream, static_cast<const char*>(a.in), static_cast<char*>(a.out), g);
    return hipGetLastError();
}


// ---------------------------------------------------------------------------
// Ulysses Anything ("Context parallelism" page, Ulysses Anything Attention:
// neither the sequence nor the heads need divide by the degree).  Shard r
// holds s_r tokens, packed back to back as [B, s_r, H, d] blocks; group g is
// h_g consecutive heads:
//   seq -> head:  out_g[b][h'][off_r + s][:] = shard_r[b][s][hoff_g + h'][:]
// Grid: x over (b, s, h', unit) of one (shard, group) pair, y = shard, z = group.
struct AnyGeom {
    int64_t s_off[kAnyMaxDegree + 1];   // token offsets of the shards (s_off[P] = S)
    int64_t h_off[kAnyMaxDegree + 1];   // head offsets of the groups (h_off[P] = H)
    FastDiv f_slen[kAnyMaxDegree];      // tokens per shard (divisor 1 for an empty one)
    FastDiv f_hlen[kAnyMaxDegree];      // heads per group
    FastDiv f_upr;                      // units per row
    int64_t B, H, S, upr;
    int g0;                             // first group of this call
    int stacked;                        // output holds every group, group g at B * h_off[g] * S rows
    int direction;
};

template <int U, int UNR>
__global__ __launch_bounds__(NT) void permute_any_kernel(const char* __restrict__ in, char* __restrict__ out,
                                                         AnyGeom g) {
    typedef typename Unit<U>::T T;
    const int r = blockIdx.y;
    const int grp = g.g0 + (int)blockIdx.z;
    const uint32_t s_len = (uint32_t)(g.s_off[r + 1] - g.s_off[r]);
    const uint32_t h_len = (uint32_t)(g.h_off[grp + 1] - g.h_off[grp]);
    const uint32_t n_units = (uint32_t)g.B * s_len * h_len * (uint32_t)g.upr;
    const int64_t seq_base = g.B * g.s_off[r] * g.H * g.upr;                  // shard r's block
    const int64_t head_base = (g.stacked ? g.B * g.h_off[grp] * g.S : 0) * g.upr;  // group grp's block

    T val[UNR];
    int64_t dst[UNR];
    bool ok[UNR];
#pragma unroll
    for (int j = 0; j < UNR; ++j) {
        const uint32_t x = ((uint32_t)blockIdx.x * UNR + j) * NT + threadIdx.x;
        ok[j] = x < n_units;
        if (!ok[j]) continue;
        const uint32_t y = fdiv(x, g.f_upr);
        const uint32_t u = x - y * (uint32_t)g.upr;
        const uint32_t z = fdiv(y, g.f_hlen[grp]);
        const uint32_t hh = y - z * h_len;
        const uint32_t b = fdiv(z, g.f_slen[r]);
        const uint32_t s = z - b * s_len;
        const int64_t seq_idx = seq_base + (((int64_t)b * s_len + s) * g.H + g.h_off[grp] + hh) * g.upr + u;
        const int64_t head_idx = head_base + (((int64_t)b * h_len + hh) * g.S + g.s_off[r] + s) * g.upr + u;
        const int64_t src = g.direction == 0 ? seq_idx : head_idx;
        dst[j] = g.direction == 0 ? head_idx : seq_idx;
        if constexpr (U == 16)
            val[j] = __builtin_bit_cast(T, __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4*>(in) + src));
        else
            val[j] = reinterpret_cast<const T*>(in)[src];
    }
#pragma unroll
    for (int j = 0; j < UNR; ++j) {
        if (!ok[j]) continue;
        if constexpr (U == 16)
            __builtin_nontemporal_store(__builtin_bit_cast(nt_u32x4, val[j]), reinterpret_cast<nt_u32x4*>(out) + dst[j]);
        else
            reinterpret_cast<T*>(out)[dst[j]] = val[j];
    }
}

template <int U>
hipError_t launch_any_u(const AnyGeom& g, int P, int ngroups, uint32_t max_units, const void* in, void* out,
                        hipStream_t stream) {
    constexpr int UNR = U == 16 ? 1 : 4;
    const uint32_t nblk = (uint32_t)(((int64_t)max_units + NT * UNR - 1) / (NT * UNR));
    hipLaunchKernelGGL((permute_any_kernel<U, UNR>), dim3(nblk, (unsigned)P, (unsigned)ngroups), dim3(NT), 0,
                       stream, static_cast<const char*>(in), static_cast<char*>(out), g);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_ulysses_permute(const PermuteArgs& a, hipStream_t stream) {
    const int64_t row_bytes = a.d * a.elem_bytes;
    int U = 16;
    while (U > 1 && row_bytes % U != 0) U >>= 1;
    const int64_t upr = row_bytes / U;
    const int64_t hp = a.H / a.groups;
    const int64_t n_units = a.B * a.S_local * hp * upr;
    if (n_units <= 0) return hipSuccess;
    if (n_units >= (int64_t(1) << 31) || upr >= (int64_t(1) << 31) || a.S_local >= (int64_t(1) << 31))
        return hipErrorInvalidValue;
    PermGeom g;
    g.upr = make_fastdiv((uint32_t)upr);
    g.hp = make_fastdiv((uint32_t)hp);
    g.s_loc = make_fastdiv((uint32_t)a.S_local);
    g.n_units = (uint32_t)n_units;
    g.B = a.B;
    g.S_loc = a.S_local;
    g.H = a.H;
    g.S = a.S_local * a.degree;
    g.hpv = hp;
    g.uprv = upr;
    g.g0 = a.group < 0 ? 0 : a.group;
    g.direction = a.direction;
    g.P = a.degree;
    g.rot = a.direction == 0 ? a.rot : 0;
    const int ngroups = a.group < 0 ? a.groups : 1;
    switch (U) {
        case 16: return launch_u<16>(a, g, ngroups, stream);
        case 8: return launch_u<8>(a, g, ngroups, stream);
        case 4: return launch_u<4>(a, g, ngroups, stream);
        case 2: return launch_u<2>(a, g, ngroups, stream);
        default: return launch_u<1>(a, g, ngroups, stream);
    }
}

}  // namespace cpattn

namespace cpattn {

hipError_t launch_ulysses_anything_permute(const AnyPermuteArgs& a, hipStream_t stream) {
    const int P = a.degree;
    if (P < 1 || P > kAnyMaxDegree) return hipErrorInvalidValue;
    const int64_t row_bytes = a.d * a.elem_bytes;
    int U = 16;
    while (U > 1 && row_bytes % U != 0) U >>= 1;
    AnyGeom g{};
    g.s_off[0] = 0;
    g.h_off[0] = 0;
    for (int i = 0; i < P; ++i) {
        g.s_off[i + 1] = g.s_off[i] + a.seq_lens[i];
        g.h_off[i + 1] = g.h_off[i] + a.head_lens[i];
    }
    g.upr = row_bytes / U;
    g.B = a.B;
    g.H = a.H;
    g.S = g.s_off[P];
    g.f_upr = make_fastdiv((uint32_t)g.upr);
    int64_t max_s = 0, max_h = 0;
    for (int i = 0; i < P; ++i) {
        g.f_slen[i] = make_fastdiv((uint32_t)(a.seq_lens[i] > 0 ? a.seq_lens[i] : 1));
        g.f_hlen[i] = make_fastdiv((uint32_t)(a.head_lens[i] > 0 ? a.head_lens[i] : 1));
        max_s = a.seq_lens[i] > max_s ? a.seq_lens[i] : max_s;
    }
    const int ngroups = a.group < 0 ? P : 1;
    g.g0 = a.group < 0 ? 0 : a.group;
    for (int i = 0; i < ngroups; ++i) max_h = a.head_lens[g.g0 + i] > max_h ? a.head_lens[g.g0 + i] : max_h;
    g.stacked = a.group < 0 ? 1 : 0;
    g.direction = a.direction;
    const int64_t max_units = a.B * max_s * max_h * g.upr;
    if (max_units <= 0) return hipSuccess;
    if (max_units >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    switch (U) {
        case 16: return launch_any_u<16>(g, P, ngroups, (uint32_t)max_units, a.in, a.out, stream);
        case 8: return launch_any_u<8>(g, P, ngroups, (uint32_t)max_units, a.in, a.out, stream);
        case 4: return launch_any_u<4>(g, P, ngroups, (uint32_t)max_units, a.in, a.out, stream);
        case 2: return launch_any_u<2>(g, P, ngroups, (uint32_t)max_units, a.in, a.out, stream);
        default: return launch_any_u<1>(g, P, ngroups, (uint32_t)max_units, a.in, a.out, stream);
    }
}

}  // namespace cpattn
