// Sanitizer driver for the library's host relayout (iqk_relayout.cpp and
// iqk_status.cpp, built here with g++ and AddressSanitizer /
// UndefinedBehaviorSanitizer by tests/test_sanitizers.py): round trips of
// random wires for every member over several widths and row counts, the
// plane offsets, and every refusal path.  Exit status 0 and "ok" on success.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/iqk.h"

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint8_t next_byte() {  // xorshift64*: input bytes only
    g_state ^= g_state >> 12;
    g_state ^= g_state << 25;
    g_state ^= g_state >> 27;
    return (uint8_t)((g_state * 0x2545F4914F6CDD1Dull) >> 56);
}

#define CHECK(c)                                                       \
    do {                                                               \
        if (!(c)) {                                                    \
            std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            return 1;                                                  \
        }                                                              \
    } while (0)

int main() {
    struct Case {
        int fmt;
        int64_t n, rows;
    };
    const Case cases[] = {{IQK_IQ2_KS, 256, 3},  {IQK_IQ2_KS, 512, 33}, {IQK_IQ2_KS, 4096, 70},
                          {IQK_IQ2_K, 256, 1},   {IQK_IQ2_K, 768, 40},  {IQK_IQ2_K, 4096, 67},
                          {IQK_IQ1_S_R4, 32, 4}, {IQK_IQ1_S_R4, 96, 8}, {IQK_IQ1_S_R4, 4096, 68}};
    for (const Case& c : cases) {
        const size_t rb = iqk_row_bytes(c.fmt, c.n);
        CHECK(rb > 0);
        const size_t bytes = rb * (size_t)c.rows;
        int64_t off[5], total = -1;
        CHECK(iqk_plane_offsets(c.fmt, c.rows, c.n, off, &total) == IQK_OK);
        CHECK(total == (int64_t)bytes);
        for (int i = 0; i < 5; ++i) CHECK(off[i] == -1 || (off[i] >= 0 && off[i] < total));
        // exact-size heap buffers, so any overrun is reported
        std::vector<uint8_t> wire(bytes), s(bytes), back(bytes);
        for (auto& b : wire) b = next_byte();
        CHECK(iqk_pack_relayout(c.fmt, wire.data(), bytes, c.rows, c.n, s.data(), bytes) == IQK_OK);
        CHECK(iqk_unpack_relayout(c.fmt, s.data(), bytes, c.rows, c.n, back.data(), bytes) == IQK_OK);
        CHECK(std::memcmp(wire.data(), back.data(), bytes) == 0);
        // refusals: wrong sizes, overlap, null buffers
        CHECK(iqk_pack_relayout(c.fmt, wire.data(), bytes - 1, c.rows, c.n, s.data(), bytes) == IQK_E_SIZE);
        CHECK(iqk_pack_relayout(c.fmt, wire.data(), bytes, c.rows, c.n, s.data(), bytes + 1) == IQK_E_SIZE);
        CHECK(iqk_pack_relayout(c.fmt, wire.data(), bytes, c.rows, c.n, wire.data(), bytes) == IQK_E_ARG);
        CHECK(iqk_pack_relayout(c.fmt, nullptr, bytes, c.rows, c.n, s.data(), bytes) == IQK_E_ARG);
        CHECK(std::strlen(iqk_last_error()) > 0);
    }
    CHECK(iqk_row_bytes(IQK_IQ2_K, 100) == 0);
    CHECK(iqk_row_bytes(9, 256) == 0);
    std::vector<uint8_t> a(6 * iqk_row_bytes(IQK_IQ1_S_R4, 32)), b(a.size());
    CHECK(iqk_pack_relayout(IQK_IQ1_S_R4, a.data(), a.size(), 6, 32, b.data(), b.size()) == IQK_E_ROWS4);
    CHECK(iqk_pack_relayout(IQK_IQ2_KS, a.data(), a.size(), 1, 100, b.data(), b.size()) == IQK_E_SHAPE);
    CHECK(iqk_pack_relayout(7, a.data(), a.size(), 1, 256, b.data(), b.size()) == IQK_E_FORMAT);
    int64_t off[5], total;
    CHECK(iqk_plane_offsets(IQK_IQ2_K, -1, 256, off, &total) == IQK_E_ARG);
    std::printf("ok\n");
    return 0;
}
