// Ulysses sequence <-> head regroup: a strided-to-contiguous row copy.
//
// "Context parallelism" page, Ulysses Attention: the all-to-all leaves each
// rank with every token for a subset of heads; this kernel is the local half of
// that regroup (and of its inverse), a pure copy of d-element rows:
//   seq -> head:  out[g'][b][h'][r*S_local + s][:] = in[r][b][s][g*H/P + h'][:]
//   head -> seq:  the inverse map.
// Rows of whole 16-byte units go through an LDS-tiled transpose (below); other
// row sizes use a direct copy in units of U bytes where each thread moves UNR
// units, loads first, then stores.  Index decomposition uses multiply-high
// division by host-computed magic numbers, so the copy stays memory-bound.
// Direct grid: x over (b, s, h', unit) of one (rank, group) slice, y = rank r,
// z = group.
#include "internal.h"

#include <algorithm>

namespace cpattn {
namespace {

constexpr int NT = 256;
constexpr int UNR = 4;

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
};

template <int U>
__global__ __launch_bounds__(NT) void permute_kernel(const char* __restrict__ in, char* __restrict__ out,
                                                     PermGeom g) {
    typedef typename Unit<U>::T T;
    const int64_t r = blockIdx.y;       // sequence shard (source rank)
    const int64_t gi = blockIdx.z;      // group index within this call
    const int64_t grp = g.g0 + gi;
    const int64_t P = gridDim.y;
    // element-row strides, in units
    const int64_t seq_base = ((r * g.B) * g.S_loc * g.H + grp * g.hpv) * g.uprv;  // in [P,B,S_loc,H,row]
    const int64_t head_base = (gi * g.B * g.hpv * g.S + r * g.S_loc) * g.uprv;    // in [G,B,hp,S,row]
    (void)P;

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
        val[j] = reinterpret_cast<const T*>(in)[src];
    }
#pragma unroll
    for (int j = 0; j < UNR; ++j)
        if (ok[j]) reinterpret_cast<T*>(out)[dst[j]] = val[j];
}

// LDS-tiled variant for rows that are whole 16-byte units.  A workgroup moves
// TS consecutive tokens of one (rank, batch, group): it reads them as TS runs of
// hp*row contiguous bytes (sequence layout) into LDS, then writes each head's
// TS rows as one contiguous run (head layout) -- or the reverse for head ->
// sequence.  Global accesses are non-temporal: every byte is touched once.
// LDS holds token s's units at s * (RU + 1) + (h' * upr + u), the one-unit pad
// per token keeping the strided side of the transpose off a single bank group.
struct TiledGeom {
    FastDiv f_ru;      // units per token in the group = hp * upr
    FastDiv f_upr;     // units per row
    FastDiv f_tsu;     // TS * upr (one head's rows in a full tile)
    int64_t B, S_loc, H, S, hp, upr;
    int TS;
    int g0;
};

typedef unsigned nt_u32x4 __attribute__((ext_vector_type(4)));

template <int DIR>
__global__ __launch_bounds__(NT) void permute_tiled_kernel(const uint4* __restrict__ in, uint4* __restrict__ out,
                                                           TiledGeom g) {
    extern __shared__ uint4 tile[];
    const int64_t r = blockIdx.y;
    const int64_t gi = blockIdx.z / g.B, b = blockIdx.z % g.B;
    const int64_t grp = g.g0 + gi;
    const int64_t s0 = (int64_t)blockIdx.x * g.TS;
    const uint32_t nt = (uint32_t)min((int64_t)g.TS, g.S_loc - s0);  // tokens in this tile
    const uint32_t ru = g.f_ru.d, upr = g.f_upr.d, tsu = g.f_tsu.d;
    const uint32_t n_tok = nt * ru;                  // units, token-major walk
    const uint32_t n_head = (uint32_t)g.hp * tsu;    // units, head-major walk over a full tile
    // unit index of token (s0 + s), head h', unit u in each layout
    const int64_t seq_base = (((r * g.B + b) * g.S_loc + s0) * g.H + grp * g.hp) * g.upr;  // + s*H*upr + h'*upr + u
    const int64_t head_base = ((gi * g.B + b) * g.hp * g.S + r * g.S_loc + s0) * g.upr;   // + h'*S*upr + s*upr + u
    const int64_t seq_tok = g.H * g.upr, head_row = g.S * g.upr;

    // token-major position x -> (global unit index in the sequence layout, LDS slot)
    auto tok = [&](uint32_t x, int64_t& gidx, uint32_t& li) {
        const uint32_t s = fdiv(x, g.f_ru), rest = x - s * ru;
        gidx = seq_base + (int64_t)s * seq_tok + rest;
        li = s * (ru + 1) + rest;
    };
    // head-major position x -> (global unit index in the head layout, LDS slot); false past the tile
    auto head = [&](uint32_t x, int64_t& gidx, uint32_t& li) -> bool {
        const uint32_t hh = fdiv(x, g.f_tsu), rem = x - hh * tsu;
        const uint32_t s = fdiv(rem, g.f_upr), u = rem - s * upr;
        gidx = head_base + (int64_t)hh * head_row + (int64_t)s * g.upr + u;
        li = s * (ru + 1) + hh * upr + u;
        return s < nt;
    };

    // phase 1: global -> LDS, walking the source layout contiguously
    const uint32_t n1 = DIR == 0 ? n_tok : n_head;
    for (uint32_t base = threadIdx.x; base < n1; base += NT * UNR) {
        nt_u32x4 v[UNR];
        uint32_t li[UNR];
        bool ok[UNR];
#pragma unroll
        for (int j = 0; j < UNR; ++j) {
            const uint32_t x = base + j * NT;
            int64_t src = 0;
            ok[j] = x < n1;
            if (ok[j]) {
                if (DIR == 0) tok(x, src, li[j]);
                else ok[j] = head(x, src, li[j]);
            }
            if (ok[j]) v[j] = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4*>(in + src));
        }
#pragma unroll
        for (int j = 0; j < UNR; ++j)
            if (ok[j]) tile[li[j]] = __builtin_bit_cast(uint4, v[j]);
    }
    __syncthreads();
    // phase 2: LDS -> global, walking the destination layout contiguously
    const uint32_t n2 = DIR == 0 ? n_head : n_tok;
    for (uint32_t x = threadIdx.x; x < n2; x += NT) {
        int64_t dst;
        uint32_t li;
        bool ok = true;
        if (DIR == 0) ok = head(x, dst, li);
        else tok(x, dst, li);
        if (ok) __builtin_nontemporal_store(__builtin_bit_cast(nt_u32x4, tile[li]), reinterpret_cast<nt_u32x4*>(out + dst));
    }
}

template <int U>
hipError_t launch_u(const PermuteArgs& a, const PermGeom& g, int ngroups, hipStream_t stream) {
    const uint32_t nblk = (g.n_units + NT * UNR - 1) / (NT * UNR);
    hipLaunchKernelGGL((permute_kernel<U>), dim3(nblk, (unsigned)a.degree, (unsigned)ngroups), dim3(NT), 0, stream,
                       static_cast<const char*>(a.in), static_cast<char*>(a.out), g);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_ulysses_permute(const PermuteArgs& a, hipStream_t stream) {
    const int64_t row_bytes = a.d * a.elem_bytes;
    int U = 16;
    while (U > 1 && row_bytes % U != 0) U >>= 1;
    const int64_t upr = row_bytes / U;
    const int64_t hp = a.H / a.degree;
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
    const int ngroups = a.group < 0 ? a.degree : 1;
    // LDS-tiled transpose when rows are whole 16-byte units and a token's group fits in LDS
    constexpr int64_t kTileBytes = 32768;
    const int64_t ru = hp * upr;
    if (U == 16 && (ru + 1) * 16 <= kTileBytes && a.B * ngroups < 65536 && a.degree < 65536) {
        TiledGeom tg;
        tg.TS = (int)std::min<int64_t>(8, kTileBytes / ((ru + 1) * 16));
        tg.f_ru = make_fastdiv((uint32_t)ru);
        tg.f_upr = make_fastdiv((uint32_t)upr);
        tg.f_tsu = make_fastdiv((uint32_t)(tg.TS * upr));
        tg.B = a.B;
        tg.S_loc = a.S_local;
        tg.H = a.H;
        tg.S = a.S_local * a.degree;
        tg.hp = hp;
        tg.upr = upr;
        tg.g0 = a.group < 0 ? 0 : a.group;
        const size_t lds = (size_t)tg.TS * (ru + 1) * 16;
        const dim3 grid((unsigned)((a.S_local + tg.TS - 1) / tg.TS), (unsigned)a.degree, (unsigned)(a.B * ngroups));
        const uint4* in = static_cast<const uint4*>(a.in);
        uint4* out = static_cast<uint4*>(a.out);
        if (a.direction == 0)
            hipLaunchKernelGGL((permute_tiled_kernel<0>), grid, dim3(NT), lds, stream, in, out, tg);
        else
            hipLaunchKernelGGL((permute_tiled_kernel<1>), grid, dim3(NT), lds, stream, in, out, tg);
        return hipGetLastError();
    }
    switch (U) {
        case 16: return launch_u<16>(a, g, ngroups, stream);
        case 8: return launch_u<8>(a, g, ngroups, stream);
        case 4: return launch_u<4>(a, g, ngroups, stream);
        case 2: return launch_u<2>(a, g, ngroups, stream);
        default: return launch_u<1>(a, g, ngroups, stream);
    }
}

}  // namespace cpattn
