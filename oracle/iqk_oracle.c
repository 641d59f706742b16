/*
 * iqk_oracle.c -- plain, slow CPU oracle for the IQ_K routed-expert path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The product
 * library (dequant_iqk_moe_amd) shares no code, header, table or helper
 * with this file and must never call it.
 *
 * What it follows (all from the "mlx-iqk" package description, page 1):
 *   - "Format" section, the three stream tables (IQ2_KS, IQ2_K, IQ1_S_R4):
 *     which field lives at which granularity;
 *   - "Format" section, the two reconstruction formulas, evaluated in
 *     float32 step by step in the order the CPU dequantizer uses:
 *        w = (d * float(scale_index)) * values[4*alphabet + code]
 *        w = (d * float(2*ls + 1)) * (float(grid_value) + shift)
 *   - "Format" section, the per-row byte budgets (2 + 70n/256, 76n/256,
 *     2 + 6n/32) and the four-row groups of the IQ1_S_R4 wire;
 *   - "Surface" section: the (x, indices) switch-linear product, one output
 *     vector per (token, slot) pair, and grouping pairs by expert.
 *
 * The pages print neither the exact bit positions inside the ik block
 * structs nor the stream bit order.  The readings used here (the stand-in
 * wire layouts W1-W3 and the canonical stream layouts F1-F3) are written
 * out next to each decoder.  Equality with real ik wire bytes is unpinned.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math (no FTZ/DAZ).
 * Floating point: every reconstruction step is an IEEE float32 multiply or
 * add (no FMA contraction); products with the activation and all sums are
 * done in double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_IQ2_KS = 1, ORC_IQ2_K = 2, ORC_IQ1_S_R4 = 3 };
enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2 };

/* One decoded weight.  For the two 2-bit members: d = fp16 bits of the scale
 * that covers the weight, a = signed scale index, b = alphabet bit,
 * c = 2-bit code.  For IQ1_S_R4: d = fp16 row scale, a = ls (0..7),
 * b = shift-sign bit, c = 11-bit grid index. */
typedef struct {
    uint16_t d;
    int16_t a, b, c;
} orc_field;

/* ------------------------------------------------------------------------ */
/* IEEE-754 binary16 / bfloat16 conversions, written from the definitions.  */
/* ------------------------------------------------------------------------ */

static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float bits_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* binary16 -> binary32, exact for every input.  Normal numbers are
 * (1024 + m) * 2^(e - 25), subnormals m * 2^-24; NaN keeps its payload. */
float orc_f16_to_f32(uint16_t h) {
    uint32_t sign = (uint32_t)(h >> 15);
    uint32_t e = (h >> 10) & 0x1f;
    uint32_t m = h & 0x3ff;
    if (e == 0x1f) {
        if (m == 0) return bits_f32((sign << 31) | 0x7f800000u);
        return bits_f32((sign << 31) | 0x7f800000u | (m << 13));
    }
    double mag = (e == 0) ? ldexp((double)m, -24) : ldexp((double)(1024 + m), (int)e - 25);
    float r = (float)mag; /* exact: at most 11 significant bits */
    return sign ? -r : r;
}

/* Round a non-negative finite double q to the nearest integer, ties to even. */
static double round_half_even(double q) {
    double fl = floor(q);
    double frac = q - fl;
    if (frac > 0.5) return fl + 1.0;
    if (frac < 0.5) return fl;
    return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

/* binary32 -> binary16, round to nearest even, overflow to infinity,
 * gradual underflow; NaN becomes a quiet NaN keeping the top payload bits. */
uint16_t orc_f32_to_f16(float f) {
    uint32_t u = f32_bits(f);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    if ((u & 0x7f800000u) == 0x7f800000u) {
        if (u & 0x007fffffu) return (uint16_t)(sign | 0x7e00u | ((u & 0x007fffffu) >> 13));
        return (uint16_t)(sign | 0x7c00u);
    }
    double a = fabs((double)f);
    if (a == 0.0) return sign;
    /* exponent of the binade that a falls in, clamped to the subnormal one */
    int e = (int)floor(log2(a));
    if (ldexp(1.0, e) > a) e -= 1;       /* guard log2 rounding */
    if (ldexp(1.0, e + 1) <= a) e += 1;
    int eq = e < -14 ? -14 : e;          /* quantum is 2^(eq-10) */
    double q = round_half_even(ldexp(a, 10 - eq));
    double r = ldexp(q, eq - 10);        /* the rounded magnitude */
    if (r >= 65536.0) return (uint16_t)(sign | 0x7c00u);
    if (r < ldexp(1.0, -14)) return (uint16_t)(sign | (uint16_t)ldexp(r, 24));
    int re = (int)floor(log2(r));
    if (ldexp(1.0, re) > r) re -= 1;
    if (ldexp(1.0, re + 1) <= r) re += 1;
    uint32_t mant = (uint32_t)(ldexp(r, 10 - re) - 1024.0);
    return (uint16_t)(sign | (uint16_t)((re + 15) << 10) | (uint16_t)mant);
}

/* binary32 -> bfloat16 (the top half of a binary32), round to nearest even on
 * the 16 discarded bits; NaN becomes a quiet NaN keeping the top payload. */
uint16_t orc_f32_to_bf16(float f) {
    uint32_t u = f32_bits(f);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu))
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t keep = u >> 16;
    uint32_t rest = u & 0xffffu;
    if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1; /* may carry into inf */
    return (uint16_t)keep;
}

/* ------------------------------------------------------------------------ */
/* Sizes                                                                     */
/* ------------------------------------------------------------------------ */

static int shape_ok(int fmt, int64_t rows, int64_t n) {
    if (rows < 0 || n <= 0) return 0;
    if (fmt == ORC_IQ2_KS || fmt == ORC_IQ2_K) return n % 256 == 0;
    if (fmt == ORC_IQ1_S_R4) return n % 32 == 0;
    return 0;
}

/* Row budgets from the "Format" section: IQ2_KS 2 + 70n/256, IQ2_K 76n/256,
 * IQ1_S_R4 2 + 6n/32 bytes.  Wire and streams spend the same bytes. */
int64_t orc_row_bytes(int fmt, int64_t n) {
    if (!shape_ok(fmt, 1, n)) return -1;
    if (fmt == ORC_IQ2_KS) return 2 + 70 * n / 256;
    if (fmt == ORC_IQ2_K) return 76 * n / 256;
    return 2 + 6 * n / 32;
}

int64_t orc_tensor_bytes(int fmt, int64_t rows, int64_t n) {
    if (!shape_ok(fmt, rows, n)) return -1;
    if (fmt == ORC_IQ1_S_R4 && rows % 4 != 0) return -1;
    return rows * orc_row_bytes(fmt, n);
}

static uint16_t rd16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static void wr16(uint8_t* p, uint16_t v) { p[0] = (uint8_t)(v & 0xff); p[1] = (uint8_t)(v >> 8); }
static int getbit(const uint8_t* base, int64_t bit) { return (base[bit >> 3] >> (bit & 7)) & 1; }
static void putbits(uint8_t* base, int64_t bit, int nbits, unsigned v) {
    for (int i = 0; i < nbits; ++i) {
        int64_t b = bit + i;
        if ((v >> i) & 1u) base[b >> 3] |= (uint8_t)(1u << (b & 7));
        else base[b >> 3] &= (uint8_t)~(1u << (b & 7));
    }
}
static unsigned getbits(const uint8_t* base, int64_t bit, int nbits) {
    unsigned v = 0;
    for (int i = 0; i < nbits; ++i) v |= (unsigned)getbit(base, bit + i) << i;
    return v;
}

/* ------------------------------------------------------------------------ */
/* Canonical streams F1-F3 ("served relayout").  Each stream is a plane      */
/* over all R rows, row-major and k-contiguous, planes in the order the      */
/* stream tables list them, no padding, bits LSB-first (so a plane read as   */
/* little-endian uint32 words has element i at bits [w*i, w*i+w) of word     */
/* i*w/32).                                                                  */
/*   IQ2_KS  qs R*n/4 | scl R*n/64 | sch R*n/256 | sex R*n/256 | dv R*2      */
/*   IQ2_K   qs R*n/4 | scl R*n/32 | sex R*n/128 | dv R*(n/256)*2            */
/*   IQ1_S_R4 qs R*n/8 | qh R*(n/32)*2 | dv R*2                              */
/* ------------------------------------------------------------------------ */

/* decode rows [r0, r0+nr) of an R-row stream tensor into fields */
int orc_decode_streams(int fmt, const uint8_t* s, int64_t R, int64_t n, int64_t r0, int64_t nr, orc_field* f) {
    if (!shape_ok(fmt, R, n) || r0 < 0 || nr < 0 || r0 + nr > R) return -1;
    for (int64_t r = r0; r < r0 + nr; ++r) {
        orc_field* fr = f + (r - r0) * n;
        if (fmt == ORC_IQ2_KS) {
            const uint8_t* qs = s;
            const uint8_t* scl = qs + R * n / 4;
            const uint8_t* sch = scl + R * n / 64;
            const uint8_t* sex = sch + R * n / 256;
            const uint8_t* dv = sex + R * n / 256;
            uint16_t d = rd16(dv + 2 * r);
            for (int64_t k = 0; k < n; ++k) {
                int64_t sb = k / 32;                       /* 32-weight sub-block */
                unsigned lo = getbits(scl, (r * n / 32 + sb) * 4, 4);
                unsigned hi = (unsigned)getbit(sch, r * n / 32 + sb);
                fr[k].d = d;
                fr[k].a = (int16_t)((int)(lo | (hi << 4)) - 16);   /* offset-16 reading */
                fr[k].b = (int16_t)getbit(sex, r * n / 32 + sb);
                fr[k].c = (int16_t)getbits(qs, (r * n + k) * 2, 2);
            }
        } else if (fmt == ORC_IQ2_K) {
            const uint8_t* qs = s;
            const uint8_t* scl = qs + R * n / 4;
            const uint8_t* sex = scl + R * n / 32;
            const uint8_t* dv = sex + R * n / 128;
            for (int64_t k = 0; k < n; ++k) {
                int64_t sb = k / 16;                       /* 16-weight sub-block */
                fr[k].d = rd16(dv + 2 * (r * (n / 256) + k / 256));
                fr[k].a = (int16_t)((int)getbits(scl, (r * n / 16 + sb) * 4, 4) - 8); /* offset 8 */
                fr[k].b = (int16_t)getbit(sex, r * n / 16 + sb);
                fr[k].c = (int16_t)getbits(qs, (r * n + k) * 2, 2);
            }
        } else {
            const uint8_t* qs = s;
            const uint8_t* qh = qs + R * n / 8;
            const uint8_t* dv = qh + R * (n / 32) * 2;
            uint16_t d = rd16(dv + 2 * r);
            for (int64_t k = 0; k < n; ++k) {
                int64_t blk = k / 32, g = k / 8, j = (k / 8) % 4;
                uint16_t h = rd16(qh + 2 * (r * (n / 32) + blk));
                unsigned lo8 = qs[r * (n / 8) + g];
                fr[k].d = d;
                fr[k].a = (int16_t)((h >> 12) & 7);        /* ls */
                fr[k].b = (int16_t)(h >> 15);              /* shift sign */
                fr[k].c = (int16_t)(lo8 | (((h >> (3 * j)) & 7u) << 8));
            }
        }
    }
    return 0;
}

/* encode all R rows of fields into canonical streams (sub-block fields are
 * taken from the first weight of each sub-block) */
int orc_encode_streams(int fmt, const orc_field* f, int64_t R, int64_t n, uint8_t* s) {
    if (!shape_ok(fmt, R, n)) return -1;
    memset(s, 0, (size_t)(R * orc_row_bytes(fmt, n)));
    for (int64_t r = 0; r < R; ++r) {
        const orc_field* fr = f + r * n;
        if (fmt == ORC_IQ2_KS) {
            uint8_t* qs = s; uint8_t* scl = qs + R * n / 4; uint8_t* sch = scl + R * n / 64;
            uint8_t* sex = sch + R * n / 256; uint8_t* dv = sex + R * n / 256;
            wr16(dv + 2 * r, fr[0].d);
            for (int64_t k = 0; k < n; ++k) putbits(qs, (r * n + k) * 2, 2, (unsigned)fr[k].c);
            for (int64_t sb = 0; sb < n / 32; ++sb) {
                unsigned raw = (unsigned)(fr[sb * 32].a + 16);
                putbits(scl, (r * n / 32 + sb) * 4, 4, raw & 15u);
                putbits(sch, r * n / 32 + sb, 1, raw >> 4);
                putbits(sex, r * n / 32 + sb, 1, (unsigned)fr[sb * 32].b);
            }
        } else if (fmt == ORC_IQ2_K) {
            uint8_t* qs = s; uint8_t* scl = qs + R * n / 4; uint8_t* sex = scl + R * n / 32;
            uint8_t* dv = sex + R * n / 128;
            for (int64_t k = 0; k < n; ++k) putbits(qs, (r * n + k) * 2, 2, (unsigned)fr[k].c);
            for (int64_t sb = 0; sb < n / 16; ++sb) {
                putbits(scl, (r * n / 16 + sb) * 4, 4, (unsigned)(fr[sb * 16].a + 8));
                putbits(sex, r * n / 16 + sb, 1, (unsigned)fr[sb * 16].b);
            }
            for (int64_t b = 0; b < n / 256; ++b) wr16(dv + 2 * (r * (n / 256) + b), fr[b * 256].d);
        } else {
            uint8_t* qs = s; uint8_t* qh = qs + R * n / 8; uint8_t* dv = qh + R * (n / 32) * 2;
            wr16(dv + 2 * r, fr[0].d);
            for (int64_t blk = 0; blk < n / 32; ++blk) {
                unsigned h = 0;
                for (int j = 0; j < 4; ++j) {
                    unsigned idx = (unsigned)fr[blk * 32 + 8 * j].c;
                    qs[r * (n / 8) + blk * 4 + j] = (uint8_t)(idx & 0xff);
                    h |= ((idx >> 8) & 7u) << (3 * j);
                }
                h |= ((unsigned)fr[blk * 32].a & 7u) << 12;
                h |= ((unsigned)fr[blk * 32].b & 1u) << 15;
                wr16(qh + 2 * (r * (n / 32) + blk), (uint16_t)h);
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Stand-in wires W1-W3: the ik block-struct budgets, one plain reading of   */
/* the field order (the pages give only the budgets and the four-row group). */
/*  W1 IQ2_KS, per row: fp16 d, then n/256 blocks of 70 B:                   */
/*     uint16 extra (bit s = alphabet of sub-block s, bit 8+s = scale high   */
/*     bit of sub-block s), uint8 scales[4] (byte i: sub-block 2i low        */
/*     nibble, 2i+1 high nibble), uint8 qs[64].                              */
/*  W2 IQ2_K, per row: n/256 blocks of 76 B: fp16 d, uint16 extra (bit s =   */
/*     alphabet of 16-weight sub-block s), uint8 scales[8] (nibbles as W1),  */
/*     uint8 qs[64].                                                         */
/*  qs in W1/W2: weight j = 128h + 32p + l of a block has its code in byte   */
/*     32h + l, bits 2p..2p+1 (the 2-bit-family interleave that is not       */
/*     k-contiguous).                                                        */
/*  W3 IQ1_S_R4, per group of four rows: fp16 d[4], then n/32 blocks of      */
/*     24 B: uint8 qs[16] (byte 4j + r = low index byte of group j of row r),*/
/*     uint16 qh[4] (qh[r] = row r).                                         */
/* ------------------------------------------------------------------------ */

static int64_t wire_qs_byte(int64_t j) { return 32 * (j / 128) + (j % 32); }
static int wire_qs_shift(int64_t j) { return (int)(2 * ((j % 128) / 32)); }

int orc_decode_wire(int fmt, const uint8_t* w, int64_t R, int64_t n, int64_t r0, int64_t nr, orc_field* f) {
    if (!shape_ok(fmt, R, n) || r0 < 0 || nr < 0 || r0 + nr > R) return -1;
    if (fmt == ORC_IQ1_S_R4 && R % 4 != 0) return -1;
    int64_t rb = orc_row_bytes(fmt, n);
    for (int64_t r = r0; r < r0 + nr; ++r) {
        orc_field* fr = f + (r - r0) * n;
        if (fmt == ORC_IQ2_KS) {
            const uint8_t* row = w + r * rb;
            uint16_t d = rd16(row);
            for (int64_t k = 0; k < n; ++k) {
                const uint8_t* blk = row + 2 + 70 * (k / 256);
                int64_t j = k % 256, sb = j / 32;
                uint16_t extra = rd16(blk);
                const uint8_t* scales = blk + 2;
                const uint8_t* qs = blk + 6;
                unsigned lo = (scales[sb / 2] >> (4 * (sb % 2))) & 15u;
                unsigned hi = (extra >> (8 + sb)) & 1u;
                fr[k].d = d;
                fr[k].a = (int16_t)((int)(lo | (hi << 4)) - 16);
                fr[k].b = (int16_t)((extra >> sb) & 1u);
                fr[k].c = (int16_t)((qs[wire_qs_byte(j)] >> wire_qs_shift(j)) & 3u);
            }
        } else if (fmt == ORC_IQ2_K) {
            const uint8_t* row = w + r * rb;
            for (int64_t k = 0; k < n; ++k) {
                const uint8_t* blk = row + 76 * (k / 256);
                int64_t j = k % 256, sb = j / 16;
                uint16_t extra = rd16(blk + 2);
                const uint8_t* scales = blk + 4;
                const uint8_t* qs = blk + 12;
                fr[k].d = rd16(blk);
                fr[k].a = (int16_t)((int)((scales[sb / 2] >> (4 * (sb % 2))) & 15u) - 8);
                fr[k].b = (int16_t)((extra >> sb) & 1u);
                fr[k].c = (int16_t)((qs[wire_qs_byte(j)] >> wire_qs_shift(j)) & 3u);
            }
        } else {
            int64_t G = r / 4, ri = r % 4;
            const uint8_t* grp = w + G * 4 * rb;
            uint16_t d = rd16(grp + 2 * ri);
            for (int64_t k = 0; k < n; ++k) {
                const uint8_t* blk = grp + 8 + 24 * (k / 32);
                int64_t j = (k % 32) / 8;
                uint16_t h = rd16(blk + 16 + 2 * ri);
                unsigned lo8 = blk[4 * j + ri];
                fr[k].d = d;
                fr[k].a = (int16_t)((h >> 12) & 7);
                fr[k].b = (int16_t)(h >> 15);
                fr[k].c = (int16_t)(lo8 | (((h >> (3 * j)) & 7u) << 8));
            }
        }
    }
    return 0;
}

int orc_encode_wire(int fmt, const orc_field* f, int64_t R, int64_t n, uint8_t* w) {
    if (!shape_ok(fmt, R, n)) return -1;
    if (fmt == ORC_IQ1_S_R4 && R % 4 != 0) return -1;
    int64_t rb = orc_row_bytes(fmt, n);
    memset(w, 0, (size_t)(R * rb));
    for (int64_t r = 0; r < R; ++r) {
        const orc_field* fr = f + r * n;
        if (fmt == ORC_IQ2_KS) {
            uint8_t* row = w + r * rb;
            wr16(row, fr[0].d);
            for (int64_t b = 0; b < n / 256; ++b) {
                uint8_t* blk = row + 2 + 70 * b;
                unsigned extra = 0;
                for (int sb = 0; sb < 8; ++sb) {
                    const orc_field* fs = fr + 256 * b + 32 * sb;
                    unsigned raw = (unsigned)(fs->a + 16);
                    extra |= ((unsigned)fs->b & 1u) << sb;
                    extra |= (raw >> 4) << (8 + sb);
                    blk[2 + sb / 2] |= (uint8_t)((raw & 15u) << (4 * (sb % 2)));
                }
                wr16(blk, (uint16_t)extra);
                for (int64_t j = 0; j < 256; ++j)
                    blk[6 + wire_qs_byte(j)] |= (uint8_t)(((unsigned)fr[256 * b + j].c & 3u) << wire_qs_shift(j));
            }
        } else if (fmt == ORC_IQ2_K) {
            uint8_t* row = w + r * rb;
            for (int64_t b = 0; b < n / 256; ++b) {
                uint8_t* blk = row + 76 * b;
                wr16(blk, fr[256 * b].d);
                unsigned extra = 0;
                for (int sb = 0; sb < 16; ++sb) {
                    const orc_field* fs = fr + 256 * b + 16 * sb;
                    extra |= ((unsigned)fs->b & 1u) << sb;
                    blk[4 + sb / 2] |= (uint8_t)(((unsigned)(fs->a + 8) & 15u) << (4 * (sb % 2)));
                }
                wr16(blk + 2, (uint16_t)extra);
                for (int64_t j = 0; j < 256; ++j)
                    blk[12 + wire_qs_byte(j)] |= (uint8_t)(((unsigned)fr[256 * b + j].c & 3u) << wire_qs_shift(j));
            }
        } else {
            int64_t G = r / 4, ri = r % 4;
            uint8_t* grp = w + G * 4 * rb;
            wr16(grp + 2 * ri, fr[0].d);
            for (int64_t blk = 0; blk < n / 32; ++blk) {
                uint8_t* bp = grp + 8 + 24 * blk;
                unsigned h = 0;
                for (int j = 0; j < 4; ++j) {
                    unsigned idx = (unsigned)fr[blk * 32 + 8 * j].c;
                    bp[4 * j + ri] = (uint8_t)(idx & 0xff);
                    h |= ((idx >> 8) & 7u) << (3 * j);
                }
                h |= ((unsigned)fr[blk * 32].a & 7u) << 12;
                h |= ((unsigned)fr[blk * 32].b & 1u) << 15;
                wr16(bp + 16 + 2 * ri, (uint16_t)h);
            }
        }
    }
    return 0;
}

/* pack = decode the wire, encode the streams; unpack = the reverse. */
int orc_pack(int fmt, const uint8_t* wire, int64_t R, int64_t n, uint8_t* streams) {
    if (!shape_ok(fmt, R, n) || (fmt == ORC_IQ1_S_R4 && R % 4)) return -1;
    orc_field* f = (orc_field*)malloc(sizeof(orc_field) * (size_t)(R * n > 0 ? R * n : 1));
    if (!f) return -2;
    int rc = orc_decode_wire(fmt, wire, R, n, 0, R, f);
    if (rc == 0) rc = orc_encode_streams(fmt, f, R, n, streams);
    free(f);
    return rc;
}

int orc_unpack(int fmt, const uint8_t* streams, int64_t R, int64_t n, uint8_t* wire) {
    if (!shape_ok(fmt, R, n) || (fmt == ORC_IQ1_S_R4 && R % 4)) return -1;
    orc_field* f = (orc_field*)malloc(sizeof(orc_field) * (size_t)(R * n > 0 ? R * n : 1));
    if (!f) return -2;
    int rc = orc_decode_streams(fmt, streams, R, n, 0, R, f);
    if (rc == 0) rc = orc_encode_wire(fmt, f, R, n, wire);
    free(f);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Reconstruction, "Format" section: every step in float32, left to right.  */
/* ------------------------------------------------------------------------ */

float orc_weight(int fmt, orc_field f, int64_t k, const float* values, const int8_t* grid) {
    float d = orc_f16_to_f32(f.d);
    if (fmt == ORC_IQ1_S_R4) {
        float scale = d * (float)(2 * f.a + 1);
        float shift = f.b ? -0.125f : 0.125f;
        float g = (float)grid[(int64_t)f.c * 8 + (k % 8)];
        return scale * (g + shift);
    }
    float dl = d * (float)f.a;
    return dl * values[4 * f.b + f.c];
}

/* dequantize rows [r0, r0+nr) of an R-row stream tensor: float32 chain, then
 * (for f16 / bf16 output) one round-to-nearest-even cast. */
int orc_dequant(int fmt, const uint8_t* s, int64_t R, int64_t n, int64_t r0, int64_t nr,
                const float* values, const int8_t* grid, int dtype, void* out) {
    if (!shape_ok(fmt, R, n) || r0 < 0 || nr < 0 || r0 + nr > R) return -1;
    orc_field* f = (orc_field*)malloc(sizeof(orc_field) * (size_t)n);
    if (!f) return -2;
    for (int64_t r = 0; r < nr; ++r) {
        orc_decode_streams(fmt, s, R, n, r0 + r, 1, f);
        for (int64_t k = 0; k < n; ++k) {
            float w = orc_weight(fmt, f[k], k, values, grid);
            int64_t i = r * n + k;
            if (dtype == ORC_F32) ((float*)out)[i] = w;
            else if (dtype == ORC_F16) ((uint16_t*)out)[i] = orc_f32_to_f16(w);
            else ((uint16_t*)out)[i] = orc_f32_to_bf16(w);
        }
    }
    free(f);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Routed-expert product ("Surface" section: y = proj(x, indices)).          */
/* ------------------------------------------------------------------------ */

/* y[t, j, o] = sum_k w_{ids[t,j]}[o, k] * x[t, slot, k] for every pair
 * (t, j), slot = 0 when x_slots == 1 and j when x_slots == k.  The expert
 * tensor is [E, out, n] stacked to R = E*out rows.  x is given as exact
 * doubles; w is the float32 reconstruction (rounded once more to bfloat16
 * when w_bf16 is set); products and the sum are in double.  A pair whose
 * expert id is outside [0, E) yields NaN. */
int orc_moe(int fmt, const uint8_t* s, int64_t E, int64_t out, int64_t n,
            const float* values, const int8_t* grid,
            const double* x, int64_t x_slots, const int32_t* ids, int64_t T, int64_t k,
            int w_bf16, double* y) {
    if (!shape_ok(fmt, E * out, n) || E <= 0 || out <= 0 || T < 0 || k <= 0) return -1;
    if (x_slots != 1 && x_slots != k) return -1;
    orc_field* f = (orc_field*)malloc(sizeof(orc_field) * (size_t)n);
    if (!f) return -2;
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t j = 0; j < k; ++j) {
            int32_t e = ids[t * k + j];
            const double* xv = x + (t * x_slots + (x_slots == 1 ? 0 : j)) * n;
            double* yv = y + (t * k + j) * out;
            for (int64_t o = 0; o < out; ++o) {
                if (e < 0 || e >= E) { yv[o] = NAN; continue; }
                orc_decode_streams(fmt, s, E * out, n, (int64_t)e * out + o, 1, f);
                double acc = 0.0;
                for (int64_t kk = 0; kk < n; ++kk) {
                    float w = orc_weight(fmt, f[kk], kk, values, grid);
                    if (w_bf16) {
                        uint32_t b = (uint32_t)orc_f32_to_bf16(w) << 16;
                        w = bits_f32(b);
                    }
                    acc += (double)w * xv[kk];
                }
                yv[o] = acc;
            }
        }
    }
    free(f);
    return 0;
}

/* Routing gather ("Surface" section: sorted pairs read each expert once).
 * counts[e] = number of pairs routed to e; offsets = exclusive prefix sum
 * (E+1 entries); perm lists pair indices t*k + j grouped by expert in
 * increasing e, and by increasing pair index inside each expert (stable).
 * Pairs with an id outside [0, E) are left out of perm; the return value
 * is the number of such pairs. */
int64_t orc_route(const int32_t* ids, int64_t P, int64_t E, int32_t* counts, int32_t* offsets, int32_t* perm) {
    for (int64_t e = 0; e < E; ++e) counts[e] = 0;
    int64_t bad = 0;
    for (int64_t p = 0; p < P; ++p) {
        if (ids[p] < 0 || ids[p] >= E) { ++bad; continue; }
        counts[ids[p]] += 1;
    }
    offsets[0] = 0;
    for (int64_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int64_t pos = 0;
    for (int64_t e = 0; e < E; ++e)
        for (int64_t p = 0; p < P; ++p)
            if (ids[p] == e) perm[pos++] = (int32_t)p;
    return bad;
}

/* element-wise array forms of the three conversions (for exhaustive sweeps) */
void orc_f16_to_f32_n(const uint16_t* h, float* out, int64_t count) {
    for (int64_t i = 0; i < count; ++i) out[i] = orc_f16_to_f32(h[i]);
}
void orc_f32_to_f16_n(const float* f, uint16_t* out, int64_t count) {
    for (int64_t i = 0; i < count; ++i) out[i] = orc_f32_to_f16(f[i]);
}
void orc_f32_to_bf16_n(const float* f, uint16_t* out, int64_t count) {
    for (int64_t i = 0; i < count; ++i) out[i] = orc_f32_to_bf16(f[i]);
}
