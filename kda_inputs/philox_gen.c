/*
 * Seeded synthetic-input generator: Philox4x32-10 counter-based RNG
 * (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3",
 * SC'11), uniforms on (0,1) and Box-Muller normals.
 *
 * This file holds random-number generation only; none of the attention
 * method's arithmetic lives here.  Stream layout: element e of a tensor drawn
 * with (seed, stream) takes word e%4 of the Philox block with counter
 * (e/4 low 32 bits, e/4 high 32 bits, 0, 0) and key (seed, stream).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

static inline void philox_round(uint32_t c[4], const uint32_t k[2]) {
    uint64_t p0 = (uint64_t)PHILOX_M0 * c[0];
    uint64_t p1 = (uint64_t)PHILOX_M1 * c[2];
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c[1] ^ k[0];
    uint32_t n2 = hi0 ^ c[3] ^ k[1];
    c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
}

/* One Philox4x32-10 block: ten rounds, key bumped by the Weyl constants between rounds. */
void kdagen_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
    uint32_t c[4] = {ctr_in[0], ctr_in[1], ctr_in[2], ctr_in[3]};
    uint32_t k[2] = {key_in[0], key_in[1]};
    for (int r = 0; r < 10; ++r) {
        if (r) { k[0] += PHILOX_W0; k[1] += PHILOX_W1; }
        philox_round(c, k);
    }
    memcpy(out, c, sizeof c);
}

static inline void block_for(uint64_t blk, uint32_t seed, uint32_t stream, uint32_t out[4]) {
    uint32_t c[4] = {(uint32_t)blk, (uint32_t)(blk >> 32), 0u, 0u};
    uint32_t k[2] = {seed, stream};
    kdagen_philox4x32_10(c, k, out);
}

/* Raw 32-bit words for elements [first, first+n). */
void kdagen_raw_u32(uint32_t seed, uint32_t stream, uint64_t first, uint64_t n, uint32_t* out) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < (int64_t)n; ++i) {
        uint64_t e = first + (uint64_t)i;
        uint32_t w[4];
        block_for(e >> 2, seed, stream, w);
        out[i] = w[e & 3];
    }
}

static inline double to_unit(uint32_t x) { return ((double)x + 0.5) * (1.0 / 4294967296.0); }

/* The four normals of one Philox block: words (0,1) and (2,3) each give a Box-Muller pair. */
static inline void block_normals(uint64_t blk, uint32_t seed, uint32_t stream, double z[4]) {
    const double two_pi = 6.283185307179586476925286766559;
    uint32_t w[4];
    block_for(blk, seed, stream, w);
    for (int pair = 0; pair < 2; ++pair) {
        double u1 = to_unit(w[2 * pair]), u2 = to_unit(w[2 * pair + 1]);
        double rad = sqrt(-2.0 * log(u1));
        z[2 * pair] = rad * cos(two_pi * u2);
        z[2 * pair + 1] = rad * sin(two_pi * u2);
    }
}

/* Uniforms on the open interval (0,1), in double, for elements [first, first+n). */
void kdagen_uniform(uint32_t seed, uint32_t stream, uint64_t first, uint64_t n, double* out) {
    if (n == 0) return;
    uint64_t b0 = first >> 2, b1 = (first + n - 1) >> 2;
    #pragma omp parallel for schedule(static)
    for (int64_t b = (int64_t)b0; b <= (int64_t)b1; ++b) {
        uint32_t w[4];
        block_for((uint64_t)b, seed, stream, w);
        for (int j = 0; j < 4; ++j) {
            uint64_t e = ((uint64_t)b << 2) + (uint64_t)j;
            if (e >= first && e < first + n) out[e - first] = to_unit(w[j]);
        }
    }
}

/* Standard normals (double) for elements [first, first+n). */
void kdagen_normal(uint32_t seed, uint32_t stream, uint64_t first, uint64_t n, double* out) {
    if (n == 0) return;
    uint64_t b0 = first >> 2, b1 = (first + n - 1) >> 2;
    #pragma omp parallel for schedule(static)
    for (int64_t b = (int64_t)b0; b <= (int64_t)b1; ++b) {
        double z[4];
        block_normals((uint64_t)b, seed, stream, z);
        for (int j = 0; j < 4; ++j) {
            uint64_t e = ((uint64_t)b << 2) + (uint64_t)j;
            if (e >= first && e < first + n) out[e - first] = z[j];
        }
    }
}

/* Normals times `scale`, rounded to float32, for elements [first, first+n). */
void kdagen_normal_f32(uint32_t seed, uint32_t stream, uint64_t first, uint64_t n, double scale, float* out) {
    if (n == 0) return;
    uint64_t b0 = first >> 2, b1 = (first + n - 1) >> 2;
    #pragma omp parallel for schedule(static)
    for (int64_t b = (int64_t)b0; b <= (int64_t)b1; ++b) {
        double z[4];
        block_normals((uint64_t)b, seed, stream, z);
        for (int j = 0; j < 4; ++j) {
            uint64_t e = ((uint64_t)b << 2) + (uint64_t)j;
            if (e >= first && e < first + n) out[e - first] = (float)(z[j] * scale);
        }
    }
}

/*
 * `rows` rows of `width` normals (elements r*width .. r*width+width-1 of the
 * stream), each scaled to unit Euclidean length in double and rounded to
 * float32: the recipe for query and key vectors.  width <= 4096.
 */
int kdagen_unit_rows_f32(uint32_t seed, uint32_t stream, uint64_t rows, uint32_t width, float* out) {
    if (width == 0 || width > 4096) return -1;
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < (int64_t)rows; ++r) {
        double buf[4096 + 8];
        uint64_t e0 = (uint64_t)r * width, e1 = e0 + width;
        for (uint64_t b = e0 >> 2; b <= (e1 - 1) >> 2; ++b) {
            double z[4];
            block_normals(b, seed, stream, z);
            for (int j = 0; j < 4; ++j) {
                uint64_t e = (b << 2) + (uint64_t)j;
                if (e >= e0 && e < e1) buf[e - e0] = z[j];
            }
        }
        double ss = 0.0;
        for (uint32_t c = 0; c < width; ++c) ss += buf[c] * buf[c];
        double inv = ss > 0.0 ? 1.0 / sqrt(ss) : 0.0;
        for (uint32_t c = 0; c < width; ++c) out[e0 + c] = (float)(buf[c] * inv);
    }
    return 0;
}

/* float32 -> bfloat16 bits, round to nearest even (NaN kept quiet). */
void kdagen_f32_to_bf16(const float* in, uint64_t n, uint16_t* out) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < (int64_t)n; ++i) {
        uint32_t x;
        memcpy(&x, &in[i], 4);
        if ((x & 0x7f800000u) == 0x7f800000u && (x & 0x007fffffu)) { out[i] = (uint16_t)((x >> 16) | 0x40); continue; }
        uint32_t lsb = (x >> 16) & 1u;
        x += 0x7fffu + lsb;
        out[i] = (uint16_t)(x >> 16);
    }
}

/* bfloat16 bits -> float32 (exact). */
void kdagen_bf16_to_f32(const uint16_t* in, uint64_t n, float* out) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < (int64_t)n; ++i) {
        uint32_t x = (uint32_t)in[i] << 16;
        memcpy(&out[i], &x, 4);
    }
}
