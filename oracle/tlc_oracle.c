/*
 * tlc_oracle.c -- plain, single-threaded CPU oracle of the 3LC codec.
 *
 * TEST INFRASTRUCTURE ONLY (see tlc_oracle.h).  Built with
 *   gcc -std=c11 -O2 -ffp-contract=off -fno-fast-math
 * so that every fp32 operation below is one IEEE-754 binary32 operation with
 * round-to-nearest-even and no fused multiply-add.
 *
 * The steps follow the 3LC review page, section "Proposed method", in its
 * order: (1) error accumulation and ternary quantization with a sparsity
 * multiplier, (2) quartic encoding, (3) zero-run encoding; decompression runs
 * them backwards.  Each step is written as directly as possible; nothing is
 * fused, blocked or reordered.
 */
#include "tlc_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#define ZERO_BYTE 121u  /* five ternary zeros: sum_j (0+1)*3^j = 1+3+9+27+81 */
#define RUN_MAX 14u     /* codes 243..255 stand for runs of 2..14 zero bytes */
#define RUN_BASE 241u   /* a run of m (2..14) zero bytes is the code 241 + m */

static const unsigned POW3[5] = {1u, 3u, 9u, 27u, 81u};

uint64_t tlco_quartic_len(uint64_t n) { return (n + 4u) / 5u; }

static int valid_s(float s) { return isfinite(s) && s >= 1.0f && s < 2.0f; }

/* Step (1): 3-value quantization with sparsity multiplication and the
 * error-accumulation buffer (3LC page, "Proposed method", first item). */
int tlco_quantize(const float* x, float* err, uint64_t n, float s, int8_t* q, float* M_out)
{
    if (!x || !err || !q || !M_out || n == 0 || !valid_s(s)) return TLCO_ERR_INVALID_ARG;

    /* M = max |x_i + err_i| over the tensor. */
    float M = 0.0f;
    for (uint64_t i = 0; i < n; ++i) {
        float v = x[i] + err[i];
        float a = fabsf(v);
        if (a > M) M = a;
    }
    *M_out = M;

    if (M == 0.0f) {
        /* Every v_i is a zero: all codes are 0 and the error keeps v_i. */
        for (uint64_t i = 0; i < n; ++i) {
            float v = x[i] + err[i];
            q[i] = 0;
            err[i] = v;
        }
        return TLCO_OK;
    }

    float Ms = M * s;
    for (uint64_t i = 0; i < n; ++i) {
        float v = x[i] + err[i];
        float r = v / Ms;           /* IEEE fp32 division */
        float t = nearbyintf(r);    /* current rounding mode: nearest, ties to even */
        if (!(t == -1.0f || t == 0.0f || t == 1.0f)) return TLCO_ERR_RANGE;
        int qi = (int)t;
        q[i] = (int8_t)qi;
        err[i] = v - (float)qi * Ms;
    }
    return TLCO_OK;
}

/* Step (2): quartic encoding, five ternary values per byte (3LC page,
 * "Proposed method", second item).  Element i is digit i%5 of byte i/5. */
int tlco_quartic_pack(const int8_t* q, uint64_t n, uint8_t* b)
{
    if (!q || !b) return TLCO_ERR_INVALID_ARG;
    uint64_t B = tlco_quartic_len(n);
    for (uint64_t k = 0; k < B; ++k) {
        unsigned byte = 0;
        for (unsigned j = 0; j < 5; ++j) {
            uint64_t i = 5u * k + j;
            int t = (i < n) ? q[i] : 0;
            if (t < -1 || t > 1) return TLCO_ERR_RANGE;
            byte += (unsigned)(t + 1) * POW3[j];
        }
        b[k] = (uint8_t)byte;
    }
    return TLCO_OK;
}

int tlco_quartic_unpack(const uint8_t* b, uint64_t n, int8_t* q)
{
    if (!b || !q) return TLCO_ERR_INVALID_ARG;
    for (uint64_t i = 0; i < n; ++i) {
        unsigned byte = b[i / 5u];
        if (byte > 242u) return TLCO_ERR_CORRUPT;
        unsigned digit = (byte / POW3[i % 5u]) % 3u;
        q[i] = (int8_t)((int)digit - 1);
    }
    return TLCO_OK;
}

/* Step (3): zero-run encoding of runs of the zero byte (3LC page, "Proposed
 * method", third item). */
int tlco_zre_encode(const uint8_t* in, uint64_t B, uint8_t* out, uint64_t cap, uint64_t* L_out)
{
    if (!in || !out || !L_out) return TLCO_ERR_INVALID_ARG;
    uint64_t L = 0;
    uint64_t i = 0;
    while (i < B) {
        if (in[i] != ZERO_BYTE) {
            if (L >= cap) return TLCO_ERR_CAPACITY;
            out[L++] = in[i++];
            continue;
        }
        uint64_t r = 0;
        while (i < B && in[i] == ZERO_BYTE) { ++r; ++i; }
        while (r >= RUN_MAX) {
            if (L >= cap) return TLCO_ERR_CAPACITY;
            out[L++] = (uint8_t)(RUN_BASE + RUN_MAX);
            r -= RUN_MAX;
        }
        if (r == 1) {
            if (L >= cap) return TLCO_ERR_CAPACITY;
            out[L++] = (uint8_t)ZERO_BYTE;
        } else if (r >= 2) {
            if (L >= cap) return TLCO_ERR_CAPACITY;
            out[L++] = (uint8_t)(RUN_BASE + r);
        }
    }
    *L_out = L;
    return TLCO_OK;
}

int tlco_zre_decode(const uint8_t* in, uint64_t L, uint8_t* out, uint64_t B)
{
    if ((!in && L) || !out) return TLCO_ERR_INVALID_ARG;
    uint64_t pos = 0;
    for (uint64_t k = 0; k < L; ++k) {
        unsigned c = in[k];
        if (c <= 242u) {
            if (pos >= B) return TLCO_ERR_CORRUPT;
            out[pos++] = (uint8_t)c;
        } else {
            uint64_t r = c - RUN_BASE;
            if (pos + r > B) return TLCO_ERR_CORRUPT;
            for (uint64_t j = 0; j < r; ++j) out[pos++] = (uint8_t)ZERO_BYTE;
        }
    }
    return pos == B ? TLCO_OK : TLCO_ERR_CORRUPT;
}

int tlco_compress(const float* x, float* err, uint64_t n, float s,
                  uint8_t* out, uint64_t cap, uint64_t* L, float* M)
{
    if (!x || !err || !out || !L || !M || n == 0 || !valid_s(s)) return TLCO_ERR_INVALID_ARG;
    uint64_t B = tlco_quartic_len(n);
    int8_t* q = (int8_t*)malloc(n);
    uint8_t* bytes = (uint8_t*)malloc(B);
    int rc = TLCO_ERR_NOMEM;
    if (q && bytes) {
        rc = tlco_quantize(x, err, n, s, q, M);
        if (rc == TLCO_OK) rc = tlco_quartic_pack(q, n, bytes);
        if (rc == TLCO_OK) rc = tlco_zre_encode(bytes, B, out, cap, L);
    }
    free(q);
    free(bytes);
    return rc;
}

/* Shared by both decompress entry points: bytes -> ternary codes. */
static int decode_codes(const uint8_t* in, uint64_t L, uint64_t n, int8_t* q)
{
    uint64_t B = tlco_quartic_len(n);
    uint8_t* bytes = (uint8_t*)malloc(B);
    if (!bytes) return TLCO_ERR_NOMEM;
    int rc = tlco_zre_decode(in, L, bytes, B);
    if (rc == TLCO_OK) rc = tlco_quartic_unpack(bytes, n, q);
    free(bytes);
    return rc;
}

int tlco_decompress(const uint8_t* in, uint64_t L, float M, uint64_t n, float s, float* y)
{
    if (!y || n == 0 || !valid_s(s)) return TLCO_ERR_INVALID_ARG;
    int8_t* q = (int8_t*)malloc(n);
    if (!q) return TLCO_ERR_NOMEM;
    int rc = decode_codes(in, L, n, q);
    if (rc == TLCO_OK) {
        float Ms = M * s;
        for (uint64_t i = 0; i < n; ++i) y[i] = (float)q[i] * Ms;
    }
    free(q);
    return rc;
}

int tlco_decompress_accumulate(const uint8_t* in, uint64_t L, float M, uint64_t n, float s,
                               float* acc)
{
    if (!acc || n == 0 || !valid_s(s)) return TLCO_ERR_INVALID_ARG;
    int8_t* q = (int8_t*)malloc(n);
    if (!q) return TLCO_ERR_NOMEM;
    int rc = decode_codes(in, L, n, q);
    if (rc == TLCO_OK) {
        float Ms = M * s;
        for (uint64_t i = 0; i < n; ++i)
            if (q[i] != 0) acc[i] = acc[i] + (float)q[i] * Ms;
    }
    free(q);
    return rc;
}

int tlco_server_compress(const float* acc, uint32_t workers, float* err, uint64_t n, float s,
                         uint8_t* out, uint64_t cap, uint64_t* L, float* M)
{
    if (!acc || workers == 0 || n == 0) return TLCO_ERR_INVALID_ARG;
    float* avg = (float*)malloc(n * sizeof(float));
    if (!avg) return TLCO_ERR_NOMEM;
    const float w = (float)workers;
    for (uint64_t i = 0; i < n; ++i) avg[i] = acc[i] / w;  /* the mean of the workers' state changes */
    int rc = tlco_compress(avg, err, n, s, out, cap, L, M);
    free(avg);
    return rc;
}

uint64_t tlco_fixed_len(uint64_t n, int encoding)
{
    if (encoding == TLCO_ENC_QUARTIC) return tlco_quartic_len(n);
    if (encoding == TLCO_ENC_TWOBIT) return (n + 3u) / 4u;
    return 0;
}

int tlco_pack_fixed(const int8_t* q, uint64_t n, int encoding, uint8_t* out)
{
    if (!q || !out) return TLCO_ERR_INVALID_ARG;
    if (encoding == TLCO_ENC_QUARTIC) return tlco_quartic_pack(q, n, out);
    if (encoding != TLCO_ENC_TWOBIT) return TLCO_ERR_INVALID_ARG;
    uint64_t nb = tlco_fixed_len(n, encoding);
    for (uint64_t k = 0; k < nb; ++k) {
        unsigned byte = 0;
        for (unsigned j = 0; j < 4; ++j) {
            uint64_t i = 4u * k + j;
            int c = i < n ? q[i] : 0;
            byte |= (unsigned)(c + 1) << (2u * j);
        }
        out[k] = (uint8_t)byte;
    }
    return TLCO_OK;
}

int tlco_unpack_fixed(const uint8_t* in, uint64_t n, int encoding, int8_t* q)
{
    if (!in || !q) return TLCO_ERR_INVALID_ARG;
    if (encoding == TLCO_ENC_QUARTIC) return tlco_quartic_unpack(in, n, q);
    if (encoding != TLCO_ENC_TWOBIT) return TLCO_ERR_INVALID_ARG;
    uint64_t nb = tlco_fixed_len(n, encoding);
    for (uint64_t k = 0; k < nb; ++k) {
        for (unsigned j = 0; j < 4; ++j) {
            unsigned f = (in[k] >> (2u * j)) & 3u;
            if (f == 3u) return TLCO_ERR_CORRUPT;
            uint64_t i = 4u * k + j;
            if (i < n) q[i] = (int8_t)((int)f - 1);
        }
    }
    return TLCO_OK;
}

int tlco_compress_fixed(const float* x, float* err, uint64_t n, float s, int encoding,
                        uint8_t* out, uint64_t cap, float* M)
{
    if (!x || !err || !out || !M || n == 0) return TLCO_ERR_INVALID_ARG;
    uint64_t nb = tlco_fixed_len(n, encoding);
    if (nb == 0) return TLCO_ERR_INVALID_ARG;
    if (cap < nb) return TLCO_ERR_CAPACITY;
    int8_t* q = (int8_t*)malloc(n);
    if (!q) return TLCO_ERR_NOMEM;
    int rc = tlco_quantize(x, err, n, s, q, M);
    if (rc == TLCO_OK) rc = tlco_pack_fixed(q, n, encoding, out);
    free(q);
    return rc;
}

int tlco_decompress_fixed(const uint8_t* in, float M, uint64_t n, float s, int encoding, float* y)
{
    if (!in || !y || n == 0 || !valid_s(s) || tlco_fixed_len(n, encoding) == 0) return TLCO_ERR_INVALID_ARG;
    int8_t* q = (int8_t*)malloc(n);
    if (!q) return TLCO_ERR_NOMEM;
    int rc = tlco_unpack_fixed(in, n, encoding, q);
    if (rc == TLCO_OK) {
        float Ms = M * s;
        for (uint64_t i = 0; i < n; ++i) y[i] = (float)q[i] * Ms;
    }
    free(q);
    return rc;
}

/* Five-plane layout: byte k holds elements k + j*B, j = 0..4, as digit j. */
int tlco_quartic_pack_planes(const int8_t* q, uint64_t n, uint8_t* b)
{
    if (!q || !b) return TLCO_ERR_INVALID_ARG;
    uint64_t B = tlco_quartic_len(n);
    for (uint64_t k = 0; k < B; ++k) {
        unsigned byte = 0;
        for (unsigned j = 0; j < 5; ++j) {
            uint64_t i = k + (uint64_t)j * B;
            int t = (i < n) ? q[i] : 0;
            if (t < -1 || t > 1) return TLCO_ERR_RANGE;
            byte += (unsigned)(t + 1) * POW3[j];
        }
        b[k] = (uint8_t)byte;
    }
    return TLCO_OK;
}

int tlco_quartic_unpack_planes(const uint8_t* b, uint64_t n, int8_t* q)
{
    if (!b || !q) return TLCO_ERR_INVALID_ARG;
    uint64_t B = tlco_quartic_len(n);
    for (uint64_t i = 0; i < n; ++i) {
        unsigned byte = b[i % B];
        if (byte > 242u) return TLCO_ERR_CORRUPT;
        unsigned digit = (byte / POW3[i / B]) % 3u;
        q[i] = (int8_t)((int)digit - 1);
    }
    return TLCO_OK;
}

int tlco_compress_planes(const float* x, float* err, uint64_t n, float s,
                         uint8_t* out, uint64_t cap, uint64_t* L, float* M)
{
    if (!x || !err || !out || !L || !M || n == 0 || !valid_s(s)) return TLCO_ERR_INVALID_ARG;
    uint64_t B = tlco_quartic_len(n);
    int8_t* q = (int8_t*)malloc(n);
    uint8_t* bytes = (uint8_t*)malloc(B);
    int rc = TLCO_ERR_NOMEM;
    if (q && bytes) {
        rc = tlco_quantize(x, err, n, s, q, M);
        if (rc == TLCO_OK) rc = tlco_quartic_pack_planes(q, n, bytes);
        if (rc == TLCO_OK) rc = tlco_zre_encode(bytes, B, out, cap, L);
    }
    free(q);
    free(bytes);
    return rc;
}

int tlco_decompress_planes(const uint8_t* in, uint64_t L, float M, uint64_t n, float s, float* y)
{
    if (!y || n == 0 || !valid_s(s)) return TLCO_ERR_INVALID_ARG;
    uint64_t B = tlco_quartic_len(n);
    int8_t* q = (int8_t*)malloc(n);
    uint8_t* bytes = (uint8_t*)malloc(B);
    int rc = TLCO_ERR_NOMEM;
    if (q && bytes) {
        rc = tlco_zre_decode(in, L, bytes, B);
        if (rc == TLCO_OK) rc = tlco_quartic_unpack_planes(bytes, n, q);
        if (rc == TLCO_OK) {
            float Ms = M * s;
            for (uint64_t i = 0; i < n; ++i) y[i] = (float)q[i] * Ms;
        }
    }
    free(q);
    free(bytes);
    return rc;
}

/* Wire message: count 8-byte headers (L_t, M_t; little-endian), then the
 * streams in tensor order.  Bytes are written one at a time, so the layout
 * does not depend on the host's byte order. */
static void put_u32le(uint8_t* p, uint32_t v)
{
    for (unsigned k = 0; k < 4; ++k) p[k] = (uint8_t)(v >> (8u * k));
}

static uint32_t get_u32le(const uint8_t* p)
{
    uint32_t v = 0;
    for (unsigned k = 0; k < 4; ++k) v |= (uint32_t)p[k] << (8u * k);
    return v;
}

int tlco_wire_pack(const uint8_t* in, const uint64_t* offs, const uint64_t* lens, const float* M, uint32_t count,
                   uint8_t* wire, uint64_t cap, uint64_t* wire_len)
{
    if (!in || !offs || !lens || !M || !wire || !wire_len || count == 0) return TLCO_ERR_INVALID_ARG;
    uint64_t total = 8u * (uint64_t)count;
    for (uint32_t t = 0; t < count; ++t) {
        if (lens[t] > 0xFFFFFFFFu) return TLCO_ERR_INVALID_ARG;
        total += lens[t];
    }
    if (total > cap) return TLCO_ERR_CAPACITY;
    uint64_t pos = 8u * (uint64_t)count;
    for (uint32_t t = 0; t < count; ++t) {
        uint32_t mbits;
        memcpy(&mbits, &M[t], 4);
        put_u32le(wire + 8u * (uint64_t)t, (uint32_t)lens[t]);
        put_u32le(wire + 8u * (uint64_t)t + 4u, mbits);
        for (uint64_t i = 0; i < lens[t]; ++i) wire[pos + i] = in[offs[t] + i];
        pos += lens[t];
    }
    *wire_len = total;
    return TLCO_OK;
}

int tlco_wire_unpack(const uint8_t* wire, uint64_t wire_bytes, uint32_t count, const uint64_t* caps,
                     uint8_t* out, const uint64_t* offs, uint64_t* lens, float* M)
{
    if (!wire || !caps || !out || !offs || !lens || !M || count == 0) return TLCO_ERR_INVALID_ARG;
    uint64_t pos = 8u * (uint64_t)count;
    if (pos > wire_bytes) return TLCO_ERR_CORRUPT;
    for (uint32_t t = 0; t < count; ++t) {
        uint64_t L = get_u32le(wire + 8u * (uint64_t)t);
        uint32_t mbits = get_u32le(wire + 8u * (uint64_t)t + 4u);
        if (L > caps[t] || L > wire_bytes - pos) return TLCO_ERR_CORRUPT;
        memcpy(&M[t], &mbits, 4);
        lens[t] = L;
        for (uint64_t i = 0; i < L; ++i) out[offs[t] + i] = wire[pos + i];
        pos += L;
    }
    return TLCO_OK;
}
