/*
 * tlc_oracle.h -- plain, single-threaded CPU oracle of the 3LC codec.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link or
 * call this code: it exists so that tests, the smoke check and the benchmark's
 * CPU-baseline leg can check the GPU library against an obviously correct
 * implementation.  It shares no code, table or header with the GPU library.
 *
 * What is computed follows the 3LC review page ("3LC: Lightweight and
 * Effective Traffic Compression for Distributed Machine Learning"), section
 * "Proposed method": ternary quantization with a sparsity multiplier and an
 * error-accumulation buffer, quartic encoding (five ternary values per byte),
 * and zero-run encoding of runs of the all-zero byte.  The page gives no
 * formulas; the concrete definitions used here are:
 *   v_i   = x_i + err_i                         (fp32 add)
 *   M     = max_i |v_i|                         (per tensor)
 *   Ms    = M * s                               (fp32 multiply, 1 <= s < 2)
 *   q_i   = rint(v_i / Ms)   in {-1, 0, 1}      (fp32 IEEE divide, ties-to-even)
 *   err_i = v_i - q_i * Ms                      (fp32)
 *   byte_k = sum_{j<5} (q_{5k+j} + 1) * 3^j     (0..242; 121 = five zeros)
 *   zero-run encoding: a maximal run of r bytes equal to 121 is written as
 *   floor(r/14) codes 255 followed by the remainder m = r mod 14 as nothing
 *   (m = 0), the literal 121 (m = 1) or the code 241 + m (m = 2..13);
 *   every other byte is copied.  Codes 243..255 therefore mean runs of 2..14.
 *
 * Parity unpinned (conventions the page does not fix; pinned only by the
 * worked examples in tests/golden): ties of v/Ms at exactly +-0.5 round to
 * even; element i goes to byte i/5 as digit i%5 with weight 3^(i%5); a run
 * longer than 14 is split greedily from its start.
 */
#ifndef TLC_ORACLE_H
#define TLC_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    TLCO_OK = 0,
    TLCO_ERR_INVALID_ARG = 1, /* null pointer, n == 0, s outside [1,2) or not finite */
    TLCO_ERR_CAPACITY = 2,    /* output buffer smaller than needed */
    TLCO_ERR_CORRUPT = 5,     /* malformed zero-run stream, or a byte > 242 */
    TLCO_ERR_RANGE = 6,       /* a ternary code outside {-1,0,1} (cannot happen for 1 <= s < 2) */
    TLCO_ERR_NOMEM = 7
};

/* Number of quartic bytes for n values: ceil(n / 5). */
uint64_t tlco_quartic_len(uint64_t n);

/* Error accumulation + per-tensor scale + ternary quantization.
 * x[n] (read), err[n] (read, then overwritten with the new error), s.
 * Writes q[n] in {-1,0,1} and *M.  Returns TLCO_OK or an error code. */
int tlco_quantize(const float* x, float* err, uint64_t n, float s, int8_t* q, float* M);

/* Quartic encoding of q[n] into b[ceil(n/5)]; missing trailing digits are 0. */
int tlco_quartic_pack(const int8_t* q, uint64_t n, uint8_t* b);

/* Quartic decoding of b[ceil(n/5)] into q[n]; digits past n are ignored.
 * Returns TLCO_ERR_CORRUPT if a byte exceeds 242. */
int tlco_quartic_unpack(const uint8_t* b, uint64_t n, int8_t* q);

/* Zero-run encoding of in[B] into out (capacity cap bytes).  *L receives the
 * stream length (always <= B). */
int tlco_zre_encode(const uint8_t* in, uint64_t B, uint8_t* out, uint64_t cap, uint64_t* L);

/* Zero-run decoding of in[L] into out[B].  The expansion must be exactly B
 * bytes, otherwise TLCO_ERR_CORRUPT. */
int tlco_zre_decode(const uint8_t* in, uint64_t L, uint8_t* out, uint64_t B);

/* Whole compress path: quantize, pack, zero-run encode.  err is updated in
 * place; out needs tlco_quartic_len(n) bytes; *L and *M are written. */
int tlco_compress(const float* x, float* err, uint64_t n, float s,
                  uint8_t* out, uint64_t cap, uint64_t* L, float* M);

/* Whole decompress path: zero-run decode, quartic decode, dequantize.
 * y[i] = q_i * (M*s). */
int tlco_decompress(const uint8_t* in, uint64_t L, float M, uint64_t n, float s, float* y);

/* As tlco_decompress, but acc[i] += q_i * (M*s) for q_i != 0 only; elements
 * with q_i == 0 are left untouched (a -0.0 stays -0.0). */
int tlco_decompress_accumulate(const uint8_t* in, uint64_t L, float M, uint64_t n, float s,
                               float* acc);

/* Fixed-length encodings (no zero-run encoding), the ablations of the 3LC
 * page's "Proposed method" second and third items: the same quantized codes
 * written as
 *   TLCO_ENC_QUARTIC  the quartic bytes alone, ceil(n/5) bytes (1.6 bits/value);
 *   TLCO_ENC_TWOBIT   the 2-bit encoding the page compares quartic encoding
 *                     with: element i is bits 2*(i%4)..2*(i%4)+1 of byte i/4,
 *                     holding q_i + 1 (0, 1 or 2), ceil(n/4) bytes (2 bits/value);
 *                     missing trailing fields hold 1 (code 0).
 * Decoding rejects a quartic byte > 242 or a 2-bit field of 3 (TLCO_ERR_CORRUPT). */
enum { TLCO_ENC_QUARTIC = 1, TLCO_ENC_TWOBIT = 2 };
uint64_t tlco_fixed_len(uint64_t n, int encoding);
int tlco_pack_fixed(const int8_t* q, uint64_t n, int encoding, uint8_t* out);
int tlco_unpack_fixed(const uint8_t* in, uint64_t n, int encoding, int8_t* q);
int tlco_compress_fixed(const float* x, float* err, uint64_t n, float s, int encoding,
                        uint8_t* out, uint64_t cap, float* M);
int tlco_decompress_fixed(const uint8_t* in, float M, uint64_t n, float s, int encoding, float* y);

/* Model-delta direction (the 3LC page, "Proposed method", fourth item: the
 * same pipeline compresses model deltas as well as gradients).  The server's
 * state change is the mean of the workers' decoded payloads: acc holds their
 * fp32 sum (tlco_decompress_accumulate in worker order) and
 *   avg_i = acc_i / workers                     (fp32 IEEE divide)
 * is compressed exactly as tlco_compress does, with the server's own error
 * buffer err.  workers >= 1; workers == 1 is tlco_compress on acc. */
int tlco_server_compress(const float* acc, uint32_t workers, float* err, uint64_t n, float s,
                         uint8_t* out, uint64_t cap, uint64_t* L, float* M);

/* The other reading of which five values share a quartic byte (the 3LC page,
 * "Proposed method", second item, does not say): five planes of B = ceil(n/5)
 * consecutive elements, byte k holding elements k, k+B, k+2B, k+3B, k+4B,
 * element k + j*B as digit j (weight 3^j); elements past n are zero codes.
 * Quantization and zero-run encoding are those of tlco_compress.  Parity
 * unpinned by the page (a convention); pinned by the worked example in
 * tests/golden. */
int tlco_quartic_pack_planes(const int8_t* q, uint64_t n, uint8_t* b);
int tlco_quartic_unpack_planes(const uint8_t* b, uint64_t n, int8_t* q);
int tlco_compress_planes(const float* x, float* err, uint64_t n, float s,
                         uint8_t* out, uint64_t cap, uint64_t* L, float* M);
int tlco_decompress_planes(const uint8_t* in, uint64_t L, float M, uint64_t n, float s, float* y);

/* Wire message of a group of `count` tensors, what one worker would send in
 * the exchange (the 3LC page, "Proposed method": a compressed state change is
 * its scale M and its byte stream; how a group's are laid out for the wire is
 * not on the page, so this layout is a reading of this library, parity
 * unpinned by the page and pinned by the worked example in tests/golden):
 *   count headers of 8 bytes: header t = L_t as a little-endian uint32
 *   (stream bytes of tensor t), then the bits of M_t as a little-endian fp32;
 *   then the streams of tensors 0 .. count-1 back to back, no padding.
 * Total length 8 * count + sum_t L_t.
 * tlco_wire_pack: tensor t's stream is in[offs[t] .. offs[t] + lens[t]);
 *   lens[t] must be below 2^32; TLCO_ERR_CAPACITY if cap is too small.
 * tlco_wire_unpack: reads wire[0 .. wire_bytes) and writes tensor t's stream
 *   to out[offs[t] ..], lens[t] and M[t]; a length above caps[t] (the most
 *   bytes a stream of that tensor can hold) or a message shorter than its
 *   headers and streams is TLCO_ERR_CORRUPT.  Bytes after the streams are
 *   ignored. */
int tlco_wire_pack(const uint8_t* in, const uint64_t* offs, const uint64_t* lens, const float* M, uint32_t count,
                   uint8_t* wire, uint64_t cap, uint64_t* wire_len);
int tlco_wire_unpack(const uint8_t* wire, uint64_t wire_bytes, uint32_t count, const uint64_t* caps,
                     uint8_t* out, const uint64_t* offs, uint64_t* lens, float* M);

#ifdef __cplusplus
}
#endif

#endif /* TLC_ORACLE_H */
