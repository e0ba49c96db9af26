// Host-side AddressSanitizer run of the C ABI's validation paths.
//
// Every call below fails validation (or is host-only code such as the status
// strings and workspace sizing), so nothing reaches the GPU.  Host arrays the
// library reads (chunk_lens, seq_lens, head_lens) are heap blocks of exactly
// the advertised length, so any read past them is reported by the sanitizer.
// Built and run by tests/test_host_asan.py; exits non-zero on a wrong status.
// With the argument "overread" it instead makes one deliberate caller error
// (a lengths array one short) that the sanitizer must catch.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <memory>

#include "cpattn.h"

namespace {

int failures = 0;

void expect(int got, int want, int line) {
    if (got != want) {
        std::printf("line %d: status %d, expected %d (%s)\n", line, got, want, cpattn_last_error());
        ++failures;
    }
}
#define EXPECT(call, want) expect((call), (want), __LINE__)

void* fake(uintptr_t a) { return reinterpret_cast<void*>(a); }

std::unique_ptr<int64_t[]> lens(std::initializer_list<int64_t> v) {
    std::unique_ptr<int64_t[]> p(new int64_t[v.size()]);
    int i = 0;
    for (int64_t x : v) p[i++] = x;
    return p;
}

}  // namespace

int main(int argc, char** argv) {
    void* q = fake(0x10000);
    void* k = fake(0x20000000);
    void* v = fake(0x40000000);
    void* out = fake(0x60000000);
    float* lse = static_cast<float*>(fake(0x70000000));
    void* ws = fake(0x7a000000);

    if (argc > 1 && std::strcmp(argv[1], "overread") == 0) {
        // caller error on purpose: three chunks announced, two lengths given; the sanitizer
        // must report the library's read of the third (shows the library is instrumented)
        auto c = lens({8, 8});
        const size_t need = cpattn_ring_fwd_workspace_bytes(1, 2, 16, 128, 3, CPATTN_BF16);
        return cpattn_ring_fwd(q, k, v, out, lse, 1, 2, 16, 16, 128, 0.f, 3, c.get(), ws, need, CPATTN_BF16,
                               CPATTN_BF16, nullptr) == CPATTN_OK ? 0 : 2;
    }

    // block forward
    EXPECT(cpattn_block_fwd(q, k, v, out, lse, 0, 2, 16, 16, 16, 128, 0.f, CPATTN_BF16, CPATTN_FP32, nullptr),
           CPATTN_ERR_SHAPE);
    EXPECT(cpattn_block_fwd(q, k, v, out, lse, 1, 2, 16, 32, 16, 128, 0.f, CPATTN_BF16, CPATTN_FP32, nullptr),
           CPATTN_ERR_SHAPE);
    EXPECT(cpattn_block_fwd(q, k, v, out, lse, 1, 2, 16, 16, 16, 96, 0.f, CPATTN_BF16, CPATTN_FP32, nullptr),
           CPATTN_ERR_SHAPE);
    EXPECT(cpattn_block_fwd(q, k, v, out, lse, 1, 2, 16, 16, 16, 128, 0.f, 7, CPATTN_FP32, nullptr),
           CPATTN_ERR_DTYPE);
    EXPECT(cpattn_block_fwd(nullptr, k, v, out, lse, 1, 2, 16, 16, 16, 128, 0.f, CPATTN_BF16, CPATTN_FP32, nullptr),
           CPATTN_ERR_NULL);
    EXPECT(cpattn_block_fwd(q, k, v, q, lse, 1, 2, 16, 16, 16, 128, 0.f, CPATTN_BF16, CPATTN_FP32, nullptr),
           CPATTN_ERR_ALIAS);
    EXPECT(cpattn_block_fwd(q, k, v, out, lse, int64_t(1) << 40, int64_t(1) << 40, 16, 16, 16, 128, 0.f,
                            CPATTN_BF16, CPATTN_FP32, nullptr),
           CPATTN_ERR_SHAPE);
    EXPECT(cpattn_block_fwd(nullptr, nullptr, nullptr, nullptr, nullptr, 1, 2, 0, 16, 16, 128, 0.f, CPATTN_BF16,
                            CPATTN_FP32, nullptr),
           CPATTN_OK);  // empty query shard: nothing to do

    // merge
    EXPECT(cpattn_lse_merge(static_cast<float*>(out), lse, q, static_cast<float*>(k), 16, 96, CPATTN_FP32, nullptr),
           CPATTN_ERR_SHAPE);
    EXPECT(cpattn_lse_merge(nullptr, lse, q, static_cast<float*>(k), 16, 128, CPATTN_FP32, nullptr),
           CPATTN_ERR_NULL);
    EXPECT(cpattn_lse_merge(static_cast<float*>(out), lse, q, static_cast<float*>(k), 16, 128, 5, nullptr),
           CPATTN_ERR_DTYPE);

    // ring: explicit lengths are read in full before the sum is checked
    const size_t need = cpattn_ring_fwd_workspace_bytes(1, 2, 16, 128, 3, CPATTN_BF16);
    {
        auto c = lens({5, 5, 7});  // sums to 17, Skv is 16
        EXPECT(cpattn_ring_fwd(q, k, v, out, lse, 1, 2, 16, 16, 128, 0.f, 3, c.get(), ws, need, CPATTN_BF16,
                               CPATTN_BF16, nullptr),
               CPATTN_ERR_CHUNKS);
        auto n = lens({8, -1, 9});
        EXPECT(cpattn_ring_fwd(q, k, v, out, lse, 1, 2, 16, 16, 128, 0.f, 3, n.get(), ws, need, CPATTN_BF16,
                               CPATTN_BF16, nullptr),
               CPATTN_ERR_CHUNKS);
        // lengths whose int64 sum would wrap around to exactly Skv (16)
        auto w = lens({INT64_MAX, INT64_MAX, 18});
        EXPECT(cpattn_ring_fwd(q, k, v, out, lse, 1, 2, 16, 16, 128, 0.f, 3, w.get(), ws, need, CPATTN_BF16,
                               CPATTN_BF16, nullptr),
               CPATTN_ERR_CHUNKS);
        // 513 planes of one 16-row query tile: two rounds of 256 workgroups, then the leftover
        // tile's 16 key tiles split over 255 workgroups, so the step writes pieces
        // (2 slots x 256 ranges x 16 rows x 128 fp32, then 2 x 256 x 16 LSE values)
        auto g = lens({512, 256, 256});
        EXPECT(cpattn_ring_fwd(q, k, v, out, lse, 1, 513, 16, 1024, 128, 0.f, 3, g.get(), ws,
                               2 * 256 * 16 * 128 * 4 + 2 * 256 * 16 * 4 - 1, CPATTN_BF16, CPATTN_BF16, nullptr),
               CPATTN_ERR_WORKSPACE);
        EXPECT(cpattn_ring_fwd_cfg(q, k, v, out, lse, 1, 2, 16, 16, 128, 0.f, 3, c.get(), 0, nullptr, 0,
                                   CPATTN_BF16, CPATTN_BF16, nullptr),
               CPATTN_ERR_CHUNKS);
    }
    EXPECT(cpattn_ring_fwd(q, k, v, out, lse, 1, 2, 16, 18, 128, 0.f, 4, nullptr, ws, need, CPATTN_BF16,
                           CPATTN_BF16, nullptr),
           CPATTN_ERR_INDIVISIBLE);
    EXPECT(cpattn_ring_fwd(q, k, v, out, lse, 1, 2, 16, 16, 128, 0.f, 0, nullptr, ws, need, CPATTN_BF16,
                           CPATTN_BF16, nullptr),
           CPATTN_ERR_DEGREE);

    // Ulysses permute
    EXPECT(cpattn_ulysses_permute(q, out, 1, 8, 6, 64, 4, 0, 0, 2, nullptr), CPATTN_ERR_INDIVISIBLE);
    EXPECT(cpattn_ulysses_permute(q, out, 1, 8, 8, 64, 4, 4, 0, 2, nullptr), CPATTN_ERR_DEGREE);
    EXPECT(cpattn_ulysses_permute(q, out, 1, 8, 8, 64, 4, 0, 2, 2, nullptr), CPATTN_ERR_DTYPE);
    EXPECT(cpattn_ulysses_permute(q, q, 1, 8, 8, 64, 4, -1, 0, 2, nullptr), CPATTN_ERR_ALIAS);

    // Ulysses Anything: both tables are read in full before the pointers are checked
    {
        auto s = lens({5, 4, 4});
        auto h = lens({2, 2, 1});
        EXPECT(cpattn_ulysses_anything_permute(nullptr, out, 1, 5, 64, 3, s.get(), h.get(), -1, 0, 2, nullptr),
               CPATTN_ERR_NULL);
        EXPECT(cpattn_ulysses_anything_permute(q, q, 1, 5, 64, 3, s.get(), h.get(), 1, 1, 2, nullptr),
               CPATTN_ERR_ALIAS);
        EXPECT(cpattn_ulysses_anything_permute(q, out, 1, 6, 64, 3, s.get(), h.get(), 0, 0, 2, nullptr),
               CPATTN_ERR_CHUNKS);  // head counts sum to 5
        auto neg = lens({5, -4, 4});
        EXPECT(cpattn_ulysses_anything_permute(q, out, 1, 5, 64, 3, neg.get(), h.get(), 0, 0, 2, nullptr),
               CPATTN_ERR_CHUNKS);
        EXPECT(cpattn_ulysses_anything_permute(q, out, 1, 5, 64, 3, nullptr, h.get(), 0, 0, 2, nullptr),
               CPATTN_ERR_NULL);
        auto z = lens({0, 0, 0});
        EXPECT(cpattn_ulysses_anything_permute(nullptr, nullptr, 1, 5, 64, 3, z.get(), h.get(), 0, 0, 2, nullptr),
               CPATTN_OK);  // no tokens: nothing to move
    }

    // Unified
    const size_t uneed = cpattn_unified_fwd_workspace_bytes(1, 16, 8, 128, 2, 2, CPATTN_BF16, CPATTN_BF16);
    EXPECT(cpattn_unified_fwd(q, k, v, out, lse, 1, 16, 6, 128, 0.f, 2, 4, 0, 0, ws, uneed, CPATTN_BF16,
                              CPATTN_BF16, nullptr),
           CPATTN_ERR_INDIVISIBLE);
    EXPECT(cpattn_unified_fwd(q, k, v, out, lse, 1, 16, 8, 128, 0.f, 2, 2, 2, 0, ws, uneed, CPATTN_BF16,
                              CPATTN_BF16, nullptr),
           CPATTN_ERR_DEGREE);
    EXPECT(cpattn_unified_fwd(q, k, v, out, lse, 1, 16, 8, 128, 0.f, 2, 2, 0, 0, ws, uneed - 1, CPATTN_BF16,
                              CPATTN_BF16, nullptr),
           CPATTN_ERR_WORKSPACE);

    // strings: every code, out-of-range codes, and the last error text
    for (int s = -3; s < 14; ++s) {
        const char* t = cpattn_status_string(s);
        if (t == nullptr || std::strlen(t) == 0) {
            std::printf("status %d: empty string\n", s);
            ++failures;
        }
    }
    if (std::strlen(cpattn_last_error()) == 0) {
        std::printf("last error text is empty after a failing call\n");
        ++failures;
    }
    if (cpattn_version() < 100) ++failures;

    std::printf("host asan driver: %d failure(s)\n", failures);
    return failures == 0 ? 0 : 1;
}
