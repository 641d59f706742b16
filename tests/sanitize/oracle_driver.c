/* Sanitizer driver for the CPU oracle (oracle/iqk_oracle.c, built here with
 * gcc and AddressSanitizer / UndefinedBehaviorSanitizer by
 * tests/test_sanitizers.py): every entry point on random inputs with
 * exact-size heap buffers, plus the round trips and agreements the oracle
 * must satisfy (pack/unpack, wire and stream decoders, f16/bf16 output =
 * cast of the float32 output, routing a permutation).  Exit status 0 and
 * "ok" on success. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct { uint16_t d; int16_t a, b, c; } orc_field;
int64_t orc_row_bytes(int fmt, int64_t n);
int orc_pack(int fmt, const uint8_t* wire, int64_t R, int64_t n, uint8_t* streams);
int orc_unpack(int fmt, const uint8_t* streams, int64_t R, int64_t n, uint8_t* wire);
int orc_decode_streams(int fmt, const uint8_t* s, int64_t R, int64_t n, int64_t r0, int64_t nr, orc_field* f);
int orc_decode_wire(int fmt, const uint8_t* w, int64_t R, int64_t n, int64_t r0, int64_t nr, orc_field* f);
int orc_dequant(int fmt, const uint8_t* s, int64_t R, int64_t n, int64_t r0, int64_t nr, const float* values,
                const int8_t* grid, int dtype, void* out);
int orc_moe(int fmt, const uint8_t* s, int64_t E, int64_t out, int64_t n, const float* values, const int8_t* grid,
            const double* x, int64_t x_slots, const int32_t* ids, int64_t T, int64_t k, int w_bf16, double* y);
int64_t orc_route(const int32_t* ids, int64_t P, int64_t E, int32_t* counts, int32_t* offsets, int32_t* perm);
uint16_t orc_f32_to_f16(float f);
uint16_t orc_f32_to_bf16(float f);

static uint64_t g_state = 0x243F6A8885A308D3ull;
static uint32_t next_u32(void) { /* xorshift64*: inputs only */
    g_state ^= g_state >> 12;
    g_state ^= g_state << 25;
    g_state ^= g_state >> 27;
    return (uint32_t)((g_state * 0x2545F4914F6CDD1Dull) >> 32);
}

#define CHECK(c)                                                                     \
    do {                                                                             \
        if (!(c)) {                                                                  \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);           \
            return 1;                                                                \
        }                                                                            \
    } while (0)

int main(void) {
    const int fmts[3] = {1, 2, 3};
    const int64_t ns[3][2] = {{256, 512}, {256, 768}, {32, 96}};
    float values[8];
    for (int i = 0; i < 8; ++i) values[i] = (float)((int)(next_u32() % 64) - 32);
    int8_t* grid = malloc(2048 * 8);
    for (int i = 0; i < 2048 * 8; ++i) grid[i] = (int8_t)((int)(next_u32() % 3) - 1);
    for (int fi = 0; fi < 3; ++fi) {
        for (int ni = 0; ni < 2; ++ni) {
            const int fmt = fmts[fi];
            const int64_t n = ns[fi][ni], E = 3, out = 8, R = E * out;
            const int64_t bytes = R * orc_row_bytes(fmt, n);
            uint8_t* wire = malloc(bytes);
            uint8_t* s = malloc(bytes);
            uint8_t* back = malloc(bytes);
            for (int64_t i = 0; i < bytes; ++i) wire[i] = (uint8_t)next_u32();
            /* scales as small finite halves so products stay finite */
            CHECK(orc_pack(fmt, wire, R, n, s) == 0);
            CHECK(orc_unpack(fmt, s, R, n, back) == 0);
            CHECK(memcmp(wire, back, bytes) == 0);
            orc_field* fw = malloc(sizeof(orc_field) * R * n);
            orc_field* fs = malloc(sizeof(orc_field) * R * n);
            CHECK(orc_decode_wire(fmt, wire, R, n, 0, R, fw) == 0);
            CHECK(orc_decode_streams(fmt, s, R, n, 0, R, fs) == 0);
            CHECK(memcmp(fw, fs, sizeof(orc_field) * R * n) == 0);
            float* w32 = malloc(sizeof(float) * R * n);
            uint16_t* w16 = malloc(2 * R * n);
            uint16_t* wb16 = malloc(2 * R * n);
            CHECK(orc_dequant(fmt, s, R, n, 0, R, values, grid, 0, w32) == 0);
            CHECK(orc_dequant(fmt, s, R, n, 0, R, values, grid, 1, w16) == 0);
            CHECK(orc_dequant(fmt, s, R, n, 0, R, values, grid, 2, wb16) == 0);
            for (int64_t i = 0; i < R * n; ++i) {
                CHECK(w16[i] == orc_f32_to_f16(w32[i]));
                CHECK(wb16[i] == orc_f32_to_bf16(w32[i]));
            }
            /* a row window inside the tensor, and one past its end (refused) */
            CHECK(orc_dequant(fmt, s, R, n, 5, 3, values, grid, 0, w32) == 0);
            CHECK(orc_dequant(fmt, s, R, n, R - 2, 3, values, grid, 0, w32) != 0);
            const int64_t T = 4, k = 2;
            double* x = malloc(sizeof(double) * T * k * n);
            for (int64_t i = 0; i < T * k * n; ++i) x[i] = (double)((int)(next_u32() % 2001) - 1000) / 500.0;
            int32_t ids[8] = {0, 2, 1, 1, 2, -1, 0, 3};
            double* y = malloc(sizeof(double) * T * k * out);
            CHECK(orc_moe(fmt, s, E, out, n, values, grid, x, k, ids, T, k, 0, y) == 0);
            CHECK(orc_moe(fmt, s, E, out, n, values, grid, x, 1, ids, T, k, 1, y) == 0);
            CHECK(y[5 * out] != y[5 * out]); /* invalid id: NaN */
            CHECK(orc_moe(fmt, s, E, out, n, values, grid, x, 3, ids, T, k, 0, y) != 0);
            int32_t counts[3], offsets[4], perm[8];
            CHECK(orc_route(ids, 8, 3, counts, offsets, perm) == 2);
            CHECK(offsets[3] == 6);
            for (int i = 0; i + 1 < 6; ++i) CHECK(ids[perm[i]] <= ids[perm[i + 1]]);
            free(wire); free(s); free(back); free(fw); free(fs); free(w32); free(w16); free(wb16); free(x); free(y);
        }
    }
    free(grid);
    printf("ok\n");
    return 0;
}
