/*
 * tlc.h -- C ABI of the 3LC state-change codec on AMD Instinct MI355X (gfx950).
 *
 * The codec is the one described by the 3LC review page ("3LC: Lightweight
 * and Effective Traffic Compression for Distributed Machine Learning"),
 * section "Proposed method":
 *   - error accumulation + 3-value quantization with a sparsity multiplier s:
 *       v = x + err,  M = max|v| (per tensor),  q = round-half-even(v / (M*s)),
 *       err <- v - q*M*s,  q in {-1, 0, 1};
 *   - quartic encoding: five ternary values per byte, byte = sum_j (q_j+1)*3^j
 *     over five consecutive elements (first element = least significant
 *     digit), values 0..242, 121 = five zeros;
 *   - zero-run encoding: a maximal run of r bytes equal to 121 becomes
 *     floor(r/14) codes 255 and then the remainder m = r mod 14 as nothing
 *     (m = 0), a literal 121 (m = 1) or the code 241+m (m = 2..13); all other
 *     bytes are copied.  Codes 243..255 mean runs of 2..14.
 *   Decompression reverses the two encodings and dequantizes y = q*M*s, or
 *   adds q*M*s into a dense fp32 accumulator where q != 0.
 * The page calls the pipeline a drop-in transform of gradient and
 * model-delta traffic ("Proposed method", fourth and sixth items); the
 * grouped calls below apply it to many tensors in one launch sequence, the
 * tensor-fusion idea of the SparCML review page ("SparCML: High-Performance
 * Sparse Communication for Machine Learning", "Proposed method", fifth item).
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless the parameter says "host".
 *   - All device work is enqueued on `stream` (a hipStream_t; NULL = default
 *     stream) and the call returns without synchronising.  Results written to
 *     device memory (out_len, scale, status, ...) are valid once the stream
 *     reaches that point.
 *   - The library never allocates, frees or synchronises memory; the caller
 *     owns every buffer.  Scratch memory is the caller's `workspace` (device,
 *     256-byte aligned, at least the size the *_workspace_size call returns;
 *     its contents need not survive between calls), except for
 *     tlc_compress_static, whose scratch is a fixed device array.  Calls that
 *     may run at the same time need separate workspaces and separate status
 *     words.
 *   - fp32 buffers (x, err, y, acc) must be 16-byte aligned and must not
 *     alias each other or the byte streams.
 *   - Return value: TLC_OK, or a synchronous error (invalid argument, too
 *     small capacity or workspace, HIP launch failure) detected before or at
 *     launch; on such an error nothing that matters was enqueued.
 *   - `status` (device int) is set to TLC_OK by the call's first kernel and
 *     raised by later kernels if the data are bad (TLC_ERR_CORRUPT) or an
 *     internal bounded wait expired (TLC_ERR_INTERNAL).  Read it after
 *     synchronising the stream.
 *   - Limits: a tensor holds 1 .. 2^32-1 elements; 1 <= s < 2; inputs are
 *     finite and M*s does not overflow (otherwise the output is unspecified).
 */
#ifndef TLC_H
#define TLC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* tlc_stream_t; /* a hipStream_t */

enum tlc_status {
    TLC_OK = 0,
    TLC_ERR_INVALID_ARG = 1, /* null pointer, n == 0 or too large, s outside [1,2), misaligned buffer */
    TLC_ERR_CAPACITY = 2,    /* output capacity below tlc_compress_bound(n) */
    TLC_ERR_WORKSPACE = 3,   /* workspace missing, misaligned or too small */
    TLC_ERR_HIP = 4,         /* a HIP launch or runtime call failed */
    TLC_ERR_CORRUPT = 5,     /* (device status) stream does not expand to exactly ceil(n/5) bytes, or a
                                fixed-length encoding holds a byte that is no valid code */
    TLC_ERR_INTERNAL = 6,    /* (device status) a bounded inter-block wait expired */
    TLC_ERR_TOO_LARGE = 7    /* n above tlc_compress_static_max_n() (tlc_compress_static only) */
};

/* Human-readable name of a status code.  Host only; never NULL. */
const char* tlc_status_string(int code);

/* Library version string.  Host only. */
const char* tlc_version(void);

/* Bytes a compressed stream of n values can take: ceil(n/5), the quartic
 * bytes of n values ("Proposed method", second item), since the zero-run
 * encoding (third item) never makes them longer.  Host only; 0 for n == 0. */
uint64_t tlc_compress_bound(uint64_t n);

/* Workspace bytes for any single-tensor call on n values (compress,
 * decompress, accumulate): the per-tile state of the page's compress steps
 * ("Proposed method", first to third items) and of their reverse.  Host
 * only; 0 for n == 0 or n > 2^32-1. */
size_t tlc_workspace_size(uint64_t n);

/* Compress one tensor (all steps of the 3LC compress path).
 *   x[n]        fp32 state change (gradient or model delta), read only.
 *   err[n]      fp32 error-accumulation buffer, read and overwritten with the
 *               new error.  Zero it before the first step; keep one per
 *               tensor and worker across steps.
 *   s           sparsity multiplier, 1 <= s < 2.
 *   out         stream bytes, capacity out_capacity >= tlc_compress_bound(n).
 *   out_len     (device uint64) receives the stream length L <= ceil(n/5).
 *   scale       (device fp32) receives M = max|x+err|.  On entry it is read as
 *               a hint: when it still holds the previous step's M (the same
 *               buffer passed every step), the second pass reads only short
 *               per-tile lists of the values that can reach the threshold
 *               instead of the error buffer.  Any content is allowed: a
 *               missing or stale hint only costs speed, never changes a bit.
 *   status      (device int), see above. */
int tlc_compress(const float* x, float* err, uint64_t n, float s,
                 uint8_t* out, uint64_t out_capacity, uint64_t* out_len, float* scale,
                 void* workspace, size_t workspace_bytes, int* status, tlc_stream_t stream);

/* Compress for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Exactly tlc_compress, bit for bit, with the same arguments except the
 * workspace: its scratch memory is a fixed device array inside the library,
 * sized for n <= tlc_compress_static_max_n() (2^24 values; about 20 MB,
 * held by each device the library runs on until the process ends).  The call
 * allocates nothing; its first call on a device looks up that device's
 * address of the array (a symbol query).  n above the maximum returns
 * TLC_ERR_TOO_LARGE before anything is enqueued.  Every call on one device
 * shares that device's array: calls that overlap on one device (other
 * streams, other threads) race and must be ordered by the caller.  Nothing
 * in the array needs to survive or start at zero between calls. */
uint64_t tlc_compress_static_max_n(void);
int tlc_compress_static(const float* x, float* err, uint64_t n, float s,
                        uint8_t* out, uint64_t out_capacity, uint64_t* out_len, float* scale,
                        int* status, tlc_stream_t stream);

/* ---- fixed-length encodings (ablations) ------------------------------------
 * The same quantization (error buffer, M, codes) written without zero-run
 * encoding, as the 3LC page's "Proposed method" items two and three are
 * measured against each other:
 *   TLC_ENC_QUARTIC  the quartic bytes alone: byte k = sum_j (q_{5k+j}+1)*3^j,
 *                    ceil(n/5) bytes (1.6 bits per value);
 *   TLC_ENC_TWOBIT   2-bit fields, the page's point of comparison: element i
 *                    in bits 2*(i%4), 2*(i%4)+1 of byte i/4 holding q_i+1,
 *                    missing trailing fields 1, ceil(n/4) bytes (2 bits/value).
 * The length is fixed by n, so no length is returned or passed.  Decoding a
 * quartic byte above 242 or a 2-bit field of 3 sets *status =
 * TLC_ERR_CORRUPT. */
enum tlc_encoding { TLC_ENC_QUARTIC = 1, TLC_ENC_TWOBIT = 2 };

/* Bytes of a fixed-length encoding of n values; host only; 0 for n == 0,
 * n > 2^32-1 or an unknown encoding. */
uint64_t tlc_fixed_len(uint64_t n, int encoding);

/* As tlc_compress (same x, err, s, scale-as-hint, workspace, status), with
 * the codes written in `encoding` to out[0 .. tlc_fixed_len(n, encoding)). */
int tlc_compress_fixed(const float* x, float* err, uint64_t n, float s, int encoding,
                       uint8_t* out, uint64_t out_capacity, float* scale,
                       void* workspace, size_t workspace_bytes, int* status, tlc_stream_t stream);

/* y[i] = q_i * (M*s) decoded from in[0 .. tlc_fixed_len(n, encoding)).  No
 * workspace. */
int tlc_decompress_fixed(const uint8_t* in, const float* scale, uint64_t n, float s, int encoding,
                         float* y, int* status, tlc_stream_t stream);

/* Model-delta direction, server side (3LC page, "Proposed method", fourth
 * item: the same pipeline compresses model deltas as well as gradients).
 * acc[n] holds the fp32 sum of the workers' decoded payloads (for example
 * `workers` calls of tlc_decompress_accumulate on a zeroed buffer); the
 * server's state change is their mean, acc[i] / workers (fp32 IEEE divide),
 * and it is compressed exactly as tlc_compress does, with the server's own
 * error buffer err[n].  workers >= 1 (TLC_ERR_INVALID_ARG otherwise);
 * workers == 1 is tlc_compress on acc.  acc is read only; every other
 * argument is as for tlc_compress.  The divide is fused into the pass that
 * reads acc and err, so the step moves the same bytes as a compress. */
int tlc_server_compress(const float* acc, uint32_t workers, float* err, uint64_t n, float s,
                        uint8_t* out, uint64_t out_capacity, uint64_t* out_len, float* scale,
                        void* workspace, size_t workspace_bytes, int* status, tlc_stream_t stream);

/* Decompress one tensor: the reverse of the page's encodings ("Proposed
 * method", second and third items): the zero-run codes expanded back into
 * quartic bytes, each quartic byte split into its five ternary codes, and
 * y[i] = q_i * (M*s) for i < n.  The stream is in[0 .. *in_len) (device
 * length, so no host round trip is needed after tlc_compress); `in` must be
 * readable for min(*in_len, ceil(n/5)) bytes.  scale: device fp32 M.  A
 * stream that does not expand to exactly ceil(n/5) bytes sets *status =
 * TLC_ERR_CORRUPT (y is then partly written).
 *   path_hint   optional (NULL allowed): a uint32 the caller owns in pinned
 *               host memory (hipHostMalloc), which selects one of two launch
 *               sequences that give the same y bit for bit.  On entry the host
 *               reads it: 0 = sparse (zero fill of y, then the nonzero codes
 *               written over it; fastest while few 5120-value tiles hold a
 *               nonzero code), 1 = dense (every tile decoded and written once;
 *               fastest for streams longer than about 0.104 bytes per quartic
 *               byte, reached after some tens of steps of error feedback).  The
 *               call's first kernel then overwrites it with the class of this
 *               call's streams, so passing the same word every step makes each
 *               decompress follow the previous one's density without a host
 *               synchronisation.  NULL: the sparse sequence.  Memory the device
 *               cannot reach returns TLC_ERR_INVALID_ARG.  A word shared by
 *               calls in flight at once only changes which sequence runs. */
int tlc_decompress(const uint8_t* in, const uint64_t* in_len, const float* scale,
                   uint64_t n, float s, float* y,
                   void* workspace, size_t workspace_bytes, int* status, uint32_t* path_hint,
                   tlc_stream_t stream);

/* As tlc_decompress, but acc[i] += q_i * (M*s) where q_i != 0; every other
 * element of acc keeps its bits.  This is the receiving side of the page's
 * exchange of compressed state changes ("Proposed method", first and fourth
 * items: the receivers apply the decoded changes).  Applying the payloads of
 * several workers one call after another gives their sum in call order. */
int tlc_decompress_accumulate(const uint8_t* in, const uint64_t* in_len, const float* scale,
                              uint64_t n, float s, float* acc,
                              void* workspace, size_t workspace_bytes, int* status,
                              tlc_stream_t stream);

/* ---- grouped calls: many tensors, one launch sequence ----------------------
 * The tensors of a group lie back to back in one flat fp32 buffer (tensor t
 * at element offset sum_{u<t} n_u), like a gradient bucket.  M, the error
 * state and the stream are per tensor exactly as in the single-tensor calls;
 * stream t occupies out[stream_offset[t] .. + ceil(n_t/5)) (offsets are
 * 16-byte aligned; their total is info->stream_bytes).
 *
 * tlc_group_plan (host only) describes the group: it fills *info and, when
 * `table` is not NULL, writes info->table_bytes of host memory that the
 * caller copies once to device memory (any 16-byte aligned buffer) and
 * passes as d_table to the grouped calls; stream_offset (host, count
 * entries) is filled when not NULL.  The plan depends only on the sizes and
 * can be reused for every step. */
typedef struct tlc_group_info {
    uint64_t count;           /* tensors */
    uint64_t total_elems;     /* sum of sizes */
    uint64_t stream_bytes;    /* capacity of the grouped out/in buffer */
    uint64_t table_bytes;     /* bytes of the device table */
    uint64_t workspace_bytes; /* workspace for any grouped call on this group */
    uint64_t tiles;           /* internal: encode tiles */
    uint64_t chunks;          /* internal: decoder chunk slots */
    uint64_t spans;           /* internal: zero-run emit spans */
} tlc_group_info;

int tlc_group_plan(const uint64_t* sizes, uint64_t count, tlc_group_info* info,
                   void* table, size_t table_capacity, uint64_t* stream_offset);

/* Grouped compress.  x/err: flat fp32[info->total_elems]; out: bytes
 * [info->stream_bytes]; out_lens: device uint64[count]; scales: device
 * fp32[count], read on entry as per-tensor hints exactly as `scale` is in
 * tlc_compress. */
int tlc_compress_group(const tlc_group_info* info, const void* d_table,
                       const float* x, float* err, float s,
                       uint8_t* out, uint64_t* out_lens, float* scales,
                       void* workspace, size_t workspace_bytes, int* status, tlc_stream_t stream);

/* Grouped fixed-length encodings: tensor t's bytes at out[out_offsets[t]]
 * (device uint64[count], 16-byte aligned offsets recommended, ranges of
 * tlc_fixed_len(n_t, encoding) bytes that do not overlap); scales as in
 * tlc_compress_group. */
int tlc_compress_fixed_group(const tlc_group_info* info, const void* d_table, int encoding,
                             const float* x, float* err, float s, uint8_t* out,
                             const uint64_t* out_offsets, float* scales,
                             void* workspace, size_t workspace_bytes, int* status, tlc_stream_t stream);
int tlc_decompress_fixed_group(const tlc_group_info* info, const void* d_table, int encoding,
                               const uint8_t* in, const uint64_t* in_offsets, const float* scales, float s,
                               float* y, int* status, tlc_stream_t stream);

/* Grouped tlc_server_compress: acc/err flat fp32[info->total_elems], per
 * tensor mean acc / workers compressed with the server's error buffer. */
int tlc_server_compress_group(const tlc_group_info* info, const void* d_table,
                              const float* acc, uint32_t workers, float* err, float s,
                              uint8_t* out, uint64_t* out_lens, float* scales,
                              void* workspace, size_t workspace_bytes, int* status, tlc_stream_t stream);

/* Grouped decompress into flat y[info->total_elems].  in: the grouped stream
 * buffer laid out as by tlc_compress_group; in_lens: device uint64[count];
 * scales: device fp32[count]; path_hint as for tlc_decompress (the density
 * class is that of the whole group's streams). */
int tlc_decompress_group(const tlc_group_info* info, const void* d_table,
                         const uint8_t* in, const uint64_t* in_lens, const float* scales, float s,
                         float* y, void* workspace, size_t workspace_bytes, int* status,
                         uint32_t* path_hint, tlc_stream_t stream);

/* Grouped decompress-and-accumulate into flat acc[info->total_elems]. */
int tlc_decompress_accumulate_group(const tlc_group_info* info, const void* d_table,
                                    const uint8_t* in, const uint64_t* in_lens,
                                    const float* scales, float s, float* acc,
                                    void* workspace, size_t workspace_bytes, int* status,
                                    tlc_stream_t stream);

/* Decompress-and-accumulate several payloads of one group into acc in one
 * call: for p = 0 .. payloads-1 in that order, acc[i] += q_{p,i} *
 * (M_{p,t}*s) where q_{p,i} != 0; the result is bit for bit that of
 * `payloads` tlc_decompress_accumulate_group calls in order.  This is the
 * receiving side of the page's exchange ("Proposed method", first and fourth
 * items) for many senders.  Two launch sequences give the same acc:
 *   dense:  one decoder pass records where every 5120-value tile of every
 *           payload begins, then one pass reads and writes each tile of acc
 *           once (tiles no payload has a nonzero code in are skipped),
 *           adding every payload's codes for it in payload order;
 *   sparse: one decoder set-up, then one pass per payload in order, each
 *           adding only that payload's nonzero codes (fastest while the
 *           streams are near all-zero, e.g. early in error feedback).
 *   payloads       1 .. 64.
 *   in             payload p's stream buffer (laid out as by
 *                  tlc_compress_group) at in + p * in_stride; in_stride >=
 *                  info->stream_bytes and a multiple of 16 (ignored for one
 *                  payload).
 *   in_lens        device uint64[payloads * count], payload p's lengths at
 *                  in_lens + p * count.
 *   scales         device fp32[payloads * count], likewise.
 *   acc            flat fp32[info->total_elems], updated in place.
 *   workspace      at least tlc_accumulate_many_workspace_size(info,
 *                  payloads) bytes (per payload: the decoder's chunk map and
 *                  flags, and 12 bytes per 5120-value tile).
 *   path_hint      optional (NULL allowed), as for tlc_decompress: 0 = the
 *                  sparse sequence, 1 = the dense one; the call's first kernel
 *                  overwrites it with the density class of all the payloads'
 *                  streams together.  NULL: the dense sequence.
 * Errors as for tlc_decompress_accumulate_group; TLC_ERR_INVALID_ARG for
 * payloads outside 1 .. 64, a bad in_stride or a hint word the device cannot
 * reach; TLC_ERR_TOO_LARGE when payloads * count exceeds 2^31 - 1 or the
 * payloads' decoder chunks 2^32 - 1 (the workspace size is then 0). */
uint64_t tlc_accumulate_many_workspace_size(const tlc_group_info* info, uint32_t payloads);
int tlc_decompress_accumulate_many_group(const tlc_group_info* info, const void* d_table, uint32_t payloads,
                                         const uint8_t* in, uint64_t in_stride, const uint64_t* in_lens,
                                         const float* scales, float s, float* acc,
                                         void* workspace, size_t workspace_bytes, int* status,
                                         uint32_t* path_hint, tlc_stream_t stream);

/* ---- wire message of a group (the exchange between workers) -----------------
 * The 3LC page ("Proposed method", first three items) has each worker send
 * its compressed state changes: per tensor, the scale M and the zero-run
 * encoded byte stream.  A grouped stream keeps tensor t's L_t bytes at the
 * start of a slot of ceil(n_t/5) bytes, so the slots hold mostly unused
 * capacity; these calls turn a group's payload into one contiguous message of
 * the bytes alone, and back, on the device (no host synchronisation: the
 * lengths stay in device memory).  The layout is this library's, the page
 * gives none:
 *   count headers of 8 bytes, header t = L_t as a little-endian uint32, then
 *   the bits of M_t as a little-endian fp32; then the streams of tensors
 *   0 .. count-1 back to back, no padding.  Length 8*count + sum_t L_t.
 * tlc_wire_bound: the most bytes a message of the group can need,
 *   8*count + info->stream_bytes (0 for a null or empty info).
 * tlc_wire_workspace_size: workspace bytes either call needs (256-byte aligned
 *   device memory; contents need not survive between calls).
 * tlc_wire_pack_group: in, in_lens, scales as tlc_compress_group wrote them
 *   (in 16-byte aligned, info->stream_bytes long); writes the message to wire
 *   (16-byte aligned, wire_capacity >= tlc_wire_bound bytes) and its length
 *   to *wire_len (device uint64).  A length above its tensor's ceil(n/5) sets
 *   TLC_ERR_CORRUPT in *status and that stream is sent empty.
 * tlc_wire_unpack_group: reads wire[0 .. wire_bytes) (16-byte aligned; the
 *   message may be followed by other bytes) and writes each stream to its
 *   slot in out (16-byte aligned, info->stream_bytes long; the bytes after a
 *   stream in its last 16-byte word are written as 0), its length to
 *   out_lens and its M to scales, so that out/out_lens/scales decompress as
 *   the sender's payload did.  A header length above its tensor's ceil(n/5)
 *   (that stream is taken as empty), or a message longer than wire_bytes (no
 *   stream is copied) sets TLC_ERR_CORRUPT in *status.
 * Asynchronous on `stream`; no allocation.  Synchronous returns:
 * TLC_ERR_INVALID_ARG for a null or misaligned pointer or an inconsistent
 * info/table pair, TLC_ERR_CAPACITY for wire_capacity below the bound (pack)
 * or wire_bytes below 8*count (unpack), TLC_ERR_WORKSPACE for a missing,
 * misaligned or small workspace, TLC_ERR_HIP for a failed launch. */
uint64_t tlc_wire_bound(const tlc_group_info* info);
uint64_t tlc_wire_workspace_size(const tlc_group_info* info);
int tlc_wire_pack_group(const tlc_group_info* info, const void* d_table, const uint8_t* in, const uint64_t* in_lens,
                        const float* scales, uint8_t* wire, uint64_t wire_capacity, uint64_t* wire_len,
                        void* workspace, size_t workspace_bytes, int* status, tlc_stream_t stream);
/* tlc_wire_pack_ranges_group: the same payload as `ranges` messages, one per
 * consecutive range of tensors (range k: tensors cuts[k] .. cuts[k+1]-1, for
 * the owners of a sharded exchange), back to back in wire: message k is the
 * wire message of its range alone, as tlc_wire_pack_group on that range's
 * group would write it, and starts where message k-1 ends; wire_lens (device
 * uint64[ranges]) receives their lengths.  cuts: host uint32[ranges + 1],
 * cuts[0] = 0 < cuts[1] < ... < cuts[ranges] = count, 1 <= ranges <= 64
 * (TLC_ERR_INVALID_ARG otherwise).  A range's slots in `in` are the slots of
 * that range's own group shifted by a multiple of 16 bytes, so each message
 * unpacks with tlc_wire_unpack_group on the range's group plan (into a
 * buffer of its own, or into the whole group's at the range's first slot).
 * Capacity, workspace and errors as tlc_wire_pack_group. */
int tlc_wire_pack_ranges_group(const tlc_group_info* info, const void* d_table, const uint32_t* cuts, uint32_t ranges,
                               const uint8_t* in, const uint64_t* in_lens, const float* scales, uint8_t* wire,
                               uint64_t wire_capacity, uint64_t* wire_lens, void* workspace, size_t workspace_bytes,
                               int* status, tlc_stream_t stream);
/* tlc_wire_unpack_ranges_group: the inverse of tlc_wire_pack_ranges_group:
 * wire[0 .. wire_bytes) holds the `ranges` messages of consecutive tensor
 * ranges back to back (as a receiver gathers its owners' messages), and the
 * whole group's payload is written to out, out_lens and scales.  Message k's
 * headers start where message k-1 ends, so the ranges are read in order;
 * one whose headers or streams run past wire_bytes sets TLC_ERR_CORRUPT
 * (and no stream is copied), as do lengths above their tensors' ceil(n/5).
 * cuts as for tlc_wire_pack_ranges_group; capacity, workspace and the other
 * errors as tlc_wire_unpack_group. */
int tlc_wire_unpack_ranges_group(const tlc_group_info* info, const void* d_table, const uint32_t* cuts,
                                 uint32_t ranges, const uint8_t* wire, uint64_t wire_bytes, uint8_t* out,
                                 uint64_t* out_lens, float* scales, void* workspace, size_t workspace_bytes,
                                 int* status, tlc_stream_t stream);
int tlc_wire_unpack_group(const tlc_group_info* info, const void* d_table, const uint8_t* wire, uint64_t wire_bytes,
                          uint8_t* out, uint64_t* out_lens, float* scales, void* workspace, size_t workspace_bytes,
                          int* status, tlc_stream_t stream);

/* ---- five-plane byte layout (ablation) --------------------------------------
 * The 3LC page ("Proposed method", second item) packs five ternary values per
 * byte without saying which five.  The codec above takes five consecutive
 * elements.  The other reading is five planes: byte k of a tensor of n values
 * holds elements k, k+B, k+2B, k+3B, k+4B (B = ceil(n/5)) as digits 0..4.
 * That is the codec's consecutive layout applied to the tensor's elements in
 * the order p = 5k + j <- element k + jB, with zeros where k + jB >= n.  These
 * two calls move fp32 data between the two orders, tensor by tensor, so that
 * the five-plane codec is:
 *   compress:   gather(x), gather(err), tlc_compress_group on the plan of
 *               sizes 5*ceil(n_t/5), scatter(err);
 *   decompress: tlc_decompress_group on that plan, scatter(y).
 * (Zero pads change neither M nor the stream, and their error stays zero.)
 * Arguments: count tensors; device arrays src_off, dst_off and n of count
 * uint64 each: tensor t has n[t] >= 1 values; its data is read at
 * src + src_off[t] and written at dst + dst_off[t], element offsets;
 * max_n >= every n[t] (host, sizes the launch).
 *   tlc_planes_gather:  reads n[t] values, writes 5*ceil(n[t]/5) (pads 0).
 *   tlc_planes_scatter: reads 5*ceil(n[t]/5) values, writes n[t].
 * src and dst must not overlap.  Asynchronous on `stream`; no allocation.
 * Returns TLC_ERR_INVALID_ARG for a null pointer, count == 0 or above 65535,
 * or max_n == 0 or above 2^32 - 1 (an n[t] above max_n is not checked on the
 * device and is undefined), TLC_ERR_HIP for a failed launch. */
int tlc_planes_gather(const float* src, const uint64_t* src_off, float* dst, const uint64_t* dst_off,
                      const uint64_t* n, uint32_t count, uint64_t max_n, tlc_stream_t stream);
int tlc_planes_scatter(const float* src, const uint64_t* src_off, float* dst, const uint64_t* dst_off,
                       const uint64_t* n, uint32_t count, uint64_t max_n, tlc_stream_t stream);

/* ---- measurement helpers (not part of the codec) -------------------------- */

/* Streaming copy of `bytes` bytes (a multiple of 16, both pointers 16-byte
 * aligned): the achievable-HBM-bandwidth yardstick for the codec kernels. */
int tlc_copy_probe(const void* src, void* dst, uint64_t bytes, tlc_stream_t stream);

/* dst[i] = src[idx[i]] for i < n (n <= 2^32): one 4-byte read per index, the
 * scattered-read yardstick of the HBM traffic counters.  All pointers are
 * device pointers; idx entries must lie inside src (not checked). */
int tlc_gather_probe(const float* src, const uint32_t* idx, uint64_t n, float* dst, tlc_stream_t stream);

/* Kernel timing with HIP events.  While enabled, every kernel the library
 * launches is bracketed by two events recorded on the same stream.
 * tlc_profile_read synchronises those events and returns, per kernel name,
 * the number of launches and their summed duration in milliseconds, then
 * forgets them.  Host only; a diagnostic facility, not thread-safe. */
typedef struct tlc_kernel_time {
    char name[48];
    uint64_t launches;
    double total_ms;
} tlc_kernel_time;

int tlc_profile_enable(int enable);
int tlc_profile_read(tlc_kernel_time* out, int capacity, int* count);

/* Restrict the timing above to the kernel of this name (for example
 * "tlc_accum_max"), so that the events perturb the other kernels of a call
 * as little as possible; NULL brackets every kernel again.  Host only. */
int tlc_profile_only(const char* kernel_name);

#ifdef __cplusplus
}
#endif

#endif /* TLC_H */
