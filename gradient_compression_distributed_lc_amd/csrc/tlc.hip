// tlc.hip -- 3LC state-change codec for AMD Instinct MI355X (gfx950).
//
// Implements the C ABI declared in include/tlc.h.  The codec is the one of
// the 3LC review page ("3LC: Lightweight and Effective Traffic Compression
// for Distributed Machine Learning", section "Proposed method"): error
// accumulation and 3-value quantization with a sparsity multiplier, quartic
// encoding (five ternary values per byte), zero-run encoding of the all-zero
// byte, and the reverse path.  The page keeps the codec cheap with vectorised,
// byte-level operations; here every step runs in the kernels below, laid out
// for CDNA4.
//
// compress (five launches):
//   k_accum_max   the one full HBM pass: v = x + err written back to err, and
//                 the max |v| of every 512-element flat tile (128 lanes x one
//                 16-byte load each: many small blocks keep the most bytes in
//                 flight).  A tile that spans tensors keeps one partial max per
//                 tensor, in slot tile + tensor.  12 bytes per element.  Per
//                 flat tile it also keeps a short list of the elements that can
//                 reach the threshold, cut at a bound from the caller's M
//                 buffer (normally last step's M).  In the model-delta
//                 direction x is the workers' sum and is divided by their count.
//   k_tile_max    one thread per encode tile (5120 elements = 1024 quartic
//                 bytes): the tile's max from the partial maxima under it,
//                 and every tensor's M through a segmented wave max and one
//                 atomic per tensor and wave.
//   k_tile_activity  per tensor M (to the caller), M*s and the exact fp32
//                 selection threshold (select_threshold); per encode tile whose
//                 max reaches it a 32-byte job for k_quant_pack (which flat
//                 tiles reach it, whether the lists are complete).  Every other
//                 tile holds only zero codes and is summarised as a run of
//                 byte 121 without touching err.
//   k_quant_pack  one wavefront per job: codes from the lists, or from v read
//                 again in the flat tiles whose max reaches the threshold;
//                 err = v - q*M*s where q != 0; codes and a bitmap of literal
//                 bytes in LDS; zero-run encoding literal by literal into a
//                 staging slot (wave-level scans, no block barriers).
//   k_emit        spans of 256 encode tiles: block scan of the tiles' carry
//                 summaries, decoupled look-back across the tensor's spans for
//                 the span's input state, then the span's stream bytes (255
//                 runs, remainder codes, staged literals) assembled in LDS and
//                 written once.
// decompress: k_prep (decoder state; list of stream chunks; for sparse
//             streams also the zero fill of y, one 16-byte store per lane)
//             -> k_decode (one block per 4 KiB of stream bytes: expansion
//             scan + look-back across the tensor's chunks for the quartic
//             byte index; then for sparse streams only literal bytes are
//             decoded and their nonzero codes written (or, to accumulate,
//             added); for dense streams the start of every encode tile is
//             recorded)
//             -> k_expand (dense streams: one wavefront per encode tile
//             decodes it in LDS and writes it once).
// accumulate of many payloads: k_prep for all of them -> dense streams:
//             k_decode records where every payload's encode tiles begin
//             (16 KiB chunks) -> k_apply (persistent wavefronts: each tile of
//             acc through LDS once, every payload's nonzero codes added in
//             payload order); sparse streams: one add-mode k_decode launch
//             per payload, in payload order.
// fixed-length encodings (ablations: quartic bytes alone, 2-bit fields): the
//             compress kernels up to k_quant_pack, which writes each tile's
//             bytes at a fixed place over k_fixed_fill's zero-code bytes;
//             k_fixed_decode decodes one encode tile per wavefront, four per
//             block.
//
// No matrix-core work exists on this path: it is bound by HBM bandwidth.

#include <hip/hip_runtime.h>

#include <float.h>
#include <limits.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <vector>

#include "tlc.h"

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr uint32_t kFTile = 512;                  // flat tile of k_accum_max: one float4 per lane
constexpr int kAccThreads = kFTile / 4;            // lanes per k_accum_max block
constexpr uint32_t kETile = 5120;                 // encode tile: elements
constexpr uint32_t kETileBytes = kETile / 5;      // 1024 quartic bytes = 4 per lane
constexpr uint32_t kSpan = 256;                   // encode tiles per k_emit block (one per lane)
constexpr uint32_t kChunk = 4096;                 // decoder stream bytes per chunk = 16 per lane
constexpr uint32_t kWideBPL = 64;                 // stream bytes per lane of the record pass over many payloads
static_assert((kChunk & (kChunk - 1)) == 0 && ((kThreads * kWideBPL) & (kThreads * kWideBPL - 1)) == 0,
              "decoder chunks are powers of two (k_prep numbers them with shifts)");
constexpr uint32_t kZero = 121;                   // quartic byte of five zero codes
constexpr uint32_t kRunMax = 14;                  // codes 243..255 = runs of 2..14
constexpr uint32_t kRunBase = 241;
constexpr uint64_t kMaxN = 0xFFFFFFFFull;
constexpr uint32_t kSpinLimit = 1u << 20;         // bounded look-back wait (about a second)
// s_waitcnt operand that waits for every outstanding vector memory access
// and nothing else (gfx9 encoding: vmcnt 0, expcnt 7, lgkmcnt 15)
constexpr int kWaitVmem = 0x0F70;
constexpr uint32_t kPackGrid = 2048;              // most blocks of k_quant_pack
constexpr int kPackSlots = 4;                     // float4 loads per lane in one k_quant_pack batch (two flat tiles)
// Candidate lists: the first pass keeps, per flat tile, the elements that can
// still reach the threshold (see cand_bound), so that the second pass need
// not read the flat tile again.
constexpr uint32_t kCand = 64;                    // list slots per flat tile
constexpr float kCandFrac = 0.485f;               // candidate bound = hint * s * kCandFrac
constexpr uint16_t kCandNone = 0xFFFF;            // count of a flat tile without a usable list
constexpr uint32_t kCandOk = 0x80000000u;         // PackJob.fmask flag: the tensor's lists are complete
constexpr uint32_t kDecodeGrid = 2048;            // most blocks of k_decode (the grid follows the resident count)

// look-back word: 2 status bits | 62 payload bits
constexpr uint64_t kInvalid = 0, kAggregate = 1, kPrefix = 2, kPoison = 3;
constexpr uint64_t kPayloadMask = (1ull << 62) - 1;

typedef float f4 __attribute__((ext_vector_type(4)));  // vector type of the nontemporal builtins and the stores below

struct Seg {
    uint64_t elem_off;    // first element in the flat fp32 buffers
    uint32_t n;           // elements
    uint32_t etile0;      // first encode tile
    uint64_t stream_off;  // first byte of this tensor's stream slot
    uint32_t span0;       // first k_emit span
    uint32_t chunk0;      // first decoder chunk slot (capacity numbering)
};
static_assert(sizeof(Seg) == 32, "table layout");

struct TableHeader {
    uint64_t magic, count, ftiles, etiles, spans, chunks, total_elems, stream_bytes;
};
static_assert(sizeof(TableHeader) == 64, "table layout");
constexpr uint64_t kMagic = 0x34434c5433ull;  // "3TLC4"
constexpr uint32_t kStraddle = 0x80000000u;   // ftile_info flag: the flat tile spans tensors
constexpr uint32_t kMulti = 0x80000000u;      // span_seg / dec_map flag: the tensor has several spans / chunks

struct GroupView {
    const Seg* segs;            // device table, or nullptr for one tensor
    const uint32_t* ftile_info; // per flat tile: tensor of its first element | kStraddle
    const uint32_t* span_seg;   // per k_emit span: tensor
    const uint32_t* etile_seg;  // per encode tile: tensor
    uint32_t count;
    Seg one;
};

__device__ __forceinline__ Seg load_seg(const GroupView& g, uint32_t i) { return g.segs ? g.segs[i] : g.one; }

// One encode tile that can hold nonzero codes, with everything k_quant_pack
// needs to process it (written by k_tile_activity).
struct PackJob {
    uint64_t e0;     // group element offset of the tile's first element
    uint32_t et;     // encode tile index in the group (carry word, staging slot)
    uint32_t nel;    // elements in the tile
    uint32_t fmask;  // bit k: flat tile e0 / kFTile + k holds |v| >= thr; kCandOk: lists complete
    float thr;       // selection threshold of the tensor
    float ms;        // M * s of the tensor
    uint32_t gi;     // tensor
};
static_assert(sizeof(PackJob) == 32, "job layout");

// Fixed-length encodings (no zero-run encoding): the quartic bytes alone, or
// 2-bit fields (four values per byte, q+1 in bits 2*(i%4) of byte i/4).  An
// encode tile (5120 values) is fixed_tile_bytes(enc) bytes of either, at a fixed place.
struct FixedOut {
    int enc;                // 0: the 3LC stream; TLC_ENC_QUARTIC or TLC_ENC_TWOBIT
    uint8_t* out;           // compress: tensor t's bytes at out + offs[t] (offset 0 for one tensor)
    const uint64_t* offs;   // device, count entries, or nullptr for one tensor
};

__host__ __device__ __forceinline__ uint32_t fixed_tile_bytes(int enc) { return enc == TLC_ENC_TWOBIT ? 1280u : 1024u; }
__host__ __device__ __forceinline__ uint64_t fixed_len_of(uint64_t n, int enc) {
    return enc == TLC_ENC_TWOBIT ? (n + 3) / 4 : (n + 4) / 5;
}
__host__ __device__ __forceinline__ uint8_t fixed_zero_byte(int enc) { return enc == TLC_ENC_TWOBIT ? 0x55 : 121; }

__device__ __forceinline__ uint32_t quartic_len(uint32_t n) { return (uint32_t)(((uint64_t)n + 4) / 5); }
__device__ __forceinline__ uint32_t etiles_of(uint32_t n) {
    return (uint32_t)(((uint64_t)n + kETile - 1) / kETile);
}

// ---------------------------------------------------------------------------
// wave / block primitives (wave64, 4 waves per block)

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// 16-byte store of data that the kernel writes once and does not read again:
// nontemporal and at system scope (sc0 sc1 nt), so that the line is written
// through instead of being kept dirty in L2.  The policy changes the speed
// only, never the stored values.  Measured on MI355X in the compress +
// decompress round trip, against the nontemporal store alone: the zero fill
// of y 200 -> 184 us (7.3 TB/s), k_expand 247-250 -> 239-246 us, and the
// x + err -> err pass 609 -> 606-608 us.  Without the nontemporal hint the
// write-through store made k_expand alone faster still, but the compress that
// followed it paid for it (k_quant_pack 118 -> 172 us).  k_apply's acc
// write-back keeps the plain nontemporal store, which measured 1-3% faster
// there.
__device__ __forceinline__ void store_stream(f4* p, f4 v) {
    asm volatile("global_store_dwordx4 %0, %1, off sc0 sc1 nt" : : "v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

__device__ __forceinline__ float wave_max(float v) {
    for (int d = 32; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, 64));
    return v;
}

__device__ __forceinline__ uint32_t wave_excl_sum(uint32_t v, uint32_t* total) {
    const int lane = lane_id();
    uint32_t inc = v;
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t o = __shfl_up(inc, d, 64);
        if (lane >= d) inc += o;
    }
    *total = __shfl(inc, 63, 64);
    return inc - v;
}

// exclusive prefix sum over the block; *total receives the block sum
__device__ uint32_t block_excl_sum(uint32_t v, uint32_t* sm, uint32_t* total) {
    const int lane = lane_id(), w = wave_id();
    uint32_t inc = v;
    for (int d = 1; d < 64; d <<= 1) {
        uint32_t o = __shfl_up(inc, d, 64);
        if (lane >= d) inc += o;
    }
    if (lane == 63) sm[w] = inc;
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        uint32_t t = sm[i];
        before += (i < w) ? t : 0u;
        tot += t;
    }
    __syncthreads();
    *total = tot;
    return before + inc - v;
}

// exclusive scan of 62-bit payloads under an associative (not necessarily
// commutative) operation op(a, b) = "a, then b"
template <typename Op>
__device__ uint64_t block_excl_scan(uint64_t v, uint64_t identity, Op op, uint64_t* sm, uint64_t* total) {
    const int lane = lane_id(), w = wave_id();
    uint64_t inc = v;
    for (int d = 1; d < 64; d <<= 1) {
        const uint64_t o = __shfl_up(inc, d, 64);
        if (lane >= d) inc = op(o, inc);
    }
    uint64_t ex = __shfl_up(inc, 1, 64);
    if (lane == 0) ex = identity;
    if (lane == 63) sm[w] = inc;
    __syncthreads();
    uint64_t before = identity, tot = identity;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        const uint64_t t = sm[i];
        if (i < w) before = op(before, t);
        tot = op(tot, t);
    }
    __syncthreads();
    *total = tot;
    return op(before, ex);
}

__device__ __forceinline__ void publish(uint64_t* flags, uint32_t idx, uint64_t status, uint64_t payload) {
    __hip_atomic_store(flags + idx, (status << 62) | (payload & kPayloadMask), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void raise_status(int* status, int code) { atomicMax(status, code); }

// Decoupled look-back, run by the 64 lanes of wave 0 of block `idx` (idx >
// first).  Entries first..idx-1 belong to blocks that took their tickets
// earlier, so they are resident or finished and publish without waiting:
// every wait ends.  Lane l reads entry top-l; the nearest prefix ends the
// walk.  `compose(a, b)` is the payload of "a, then b".  Returns false if the
// bounded wait expires or a predecessor published poison.
template <typename Compose>
__device__ bool look_back(const uint64_t* flags, uint32_t idx, uint32_t first, uint64_t identity,
                          Compose compose, uint64_t* result) {
    const int lane = lane_id();
    uint64_t acc = identity;
    int64_t top = (int64_t)idx - 1;
    uint32_t spins = 0;
    for (;;) {
        const int64_t j = top - lane;
        const bool in = j >= (int64_t)first;
        uint64_t w;
        for (;;) {
            w = in ? __hip_atomic_load(flags + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                   : ((kPrefix << 62) | identity);
            if (__all((w >> 62) != kInvalid)) break;
            if (++spins > kSpinLimit) return false;
            __builtin_amdgcn_s_sleep(1);
        }
        if (__any((w >> 62) == kPoison)) return false;
        const uint64_t pm = __ballot((w >> 62) == kPrefix);
        const int lp = pm ? (__ffsll((unsigned long long)pm) - 1) : 64;
        uint64_t v = (lane > lp) ? identity : (w & kPayloadMask);
        // ordered reduction: a higher lane holds an older entry
        for (int d = 1; d < 64; d <<= 1) {
            const uint64_t o = __shfl_down(v, d, 64);
            if ((lane & (2 * d - 1)) == 0) v = compose(o, v);
        }
        v = __shfl(v, 0, 64);
        acc = compose(v, acc);
        if (pm) {
            *result = acc;
            return true;
        }
        top -= 64;
    }
}

// ---------------------------------------------------------------------------
// zero-run encoder carry algebra
//
// State of the encoder after a prefix of the quartic bytes: E = stream bytes
// already fixed (every completed 14-byte chunk of the pending run counts as
// its 255), r = length of the pending run of byte 121, modulo 14.  A tile
// maps states to states in one of two shapes:
//   Run(Q, p): a tile of only byte 121, l = 14Q + p bytes long:
//              (E, r) -> (E + Q + (r+p) div 14, (r+p) mod 14)
//   Lit(p, K, c): a tile whose first literal is at byte f = 14F + p, which
//              emits K - F bytes from that literal on (remainder codes inside
//              the tile, literals, completed chunks of its trailing run) and
//              leaves c = trailing run mod 14 pending:
//              (E, r) -> (E + ceil((r+p)/14) + K, c)
// Both shapes are closed under composition, so tile summaries can be scanned.
// Payload bits: 61 = Lit, 60..57 = p, 56..53 = c, 31..0 = Q or K.  Per-tile
// words also carry K - F (the staged byte count) in bits 32..42.

struct Carry {
    uint32_t K;
    uint32_t lit, p, c;
};

__device__ __forceinline__ uint64_t carry_pack(Carry a) {
    return ((uint64_t)a.lit << 61) | ((uint64_t)a.p << 57) | ((uint64_t)a.c << 53) | (uint64_t)a.K;
}
__device__ __forceinline__ Carry carry_unpack(uint64_t w) {
    Carry a;
    a.K = (uint32_t)w;
    a.lit = (uint32_t)(w >> 61) & 1u;
    a.p = (uint32_t)(w >> 57) & 15u;
    a.c = (uint32_t)(w >> 53) & 15u;
    return a;
}
__device__ __forceinline__ Carry carry_run(uint32_t len) {
    Carry a;
    a.K = len / kRunMax;
    a.lit = 0;
    a.p = len % kRunMax;
    a.c = 0;
    return a;
}
// a, then b
__device__ __forceinline__ Carry carry_compose(Carry a, Carry b) {
    Carry r;
    if (!a.lit) {
        const uint32_t t = a.p + b.p;
        r.lit = b.lit;
        r.p = t % kRunMax;
        r.K = a.K + b.K + t / kRunMax;
        r.c = b.c;
    } else if (!b.lit) {
        const uint32_t t = a.c + b.p;
        r.lit = 1;
        r.p = a.p;
        r.K = a.K + b.K + t / kRunMax;
        r.c = t % kRunMax;
    } else {
        r.lit = 1;
        r.p = a.p;
        r.K = a.K + (a.c + b.p + kRunMax - 1) / kRunMax + b.K;
        r.c = b.c;
    }
    return r;
}
// state (E, r) after applying a
__device__ __forceinline__ void carry_apply(Carry a, uint32_t E, uint32_t r, uint32_t* E2, uint32_t* r2) {
    if (!a.lit) {
        const uint32_t t = r + a.p;
        *E2 = E + a.K + t / kRunMax;
        *r2 = t % kRunMax;
    } else {
        *E2 = E + (r + a.p + kRunMax - 1) / kRunMax + a.K;
        *r2 = a.c;
    }
}
struct CarryCompose {
    __device__ uint64_t operator()(uint64_t a, uint64_t b) const {
        return carry_pack(carry_compose(carry_unpack(a), carry_unpack(b)));
    }
};
struct SumCompose {
    __device__ uint64_t operator()(uint64_t a, uint64_t b) const { return (a + b) & kPayloadMask; }
};

__device__ __forceinline__ uint8_t remainder_code(uint32_t m) {  // m = 1..13
    return (uint8_t)(m == 1 ? kZero : kRunBase + m);
}

// Candidate bound of a tensor from a hint of its M (normally the previous
// step's): an element with |v| below it has q = 0 whenever the threshold of
// this step is at least the bound, which the second pass checks before it
// relies on the lists.  Any hint is allowed: a missing or wrong one only
// sends tensors or flat tiles down the full re-read.  kCandFrac = 0.97 of
// the threshold M*s/2 at M = hint: a step whose M is within 3% below the
// hint still uses the lists.  Measured on the BERT-large set after 150 steps
// of error feedback: margins of 2-3% give the fastest step (the lists are
// written by the first pass and read by the second, so shorter lists save
// in both); 5% writes ~25% more list entries; 1% and less sends so many
// tensors down the full re-read that the second pass slows by 25-50%.
__device__ __forceinline__ float cand_bound(float hint, float s) {
    return (hint > 0.0f && hint <= FLT_MAX) ? hint * s * kCandFrac : INFINITY;
}

// Smallest float a with |v| >= a  <=>  rint(v / Ms) != 0 for fp32 v, where
// v / Ms is the correctly rounded fp32 quotient.  For |v| <= M <= Ms the
// quotient rounds to a value > 0.5 exactly when the real quotient exceeds the
// midpoint 0.5 + 2^-25 between 0.5 and the next float (the tie rounds to 0.5,
// whose significand is even).  Ms * (0.5 + 2^-25) has at most 24 + 25
// significant bits, so the fp64 product is exact, and the comparison of a
// float against it is exact too.  This replaces one fp32 division per element
// by a compare without changing any result.
__device__ float select_threshold(float m, float ms) {
    if (!(m > 0.0f)) return INFINITY;            // M == 0: every code is 0
    const double t = (double)ms * (0.5 + 0x1p-25);
    if (!(t < (double)FLT_MAX)) return INFINITY;  // M*s overflowed (unspecified input)
    float a = (float)t;
    if ((double)a <= t) a = __uint_as_float(__float_as_uint(a) + 1u);
    return a;
}

__device__ __forceinline__ int ternary(float v, float thr) {
    return fabsf(v) >= thr ? (v > 0.0f ? 1 : -1) : 0;
}

// ---------------------------------------------------------------------------
// compress kernels

__global__ __launch_bounds__(kAccThreads) void k_accum_max(GroupView g, uint64_t N, const float* __restrict__ x,
                                                        float x_div, float* __restrict__ err,
                                                        float* __restrict__ pmax, const float* __restrict__ hint,
                                                        float s, uint16_t* __restrict__ cand_cnt,
                                                        uint2* __restrict__ cand,
                                                        uint64_t* __restrict__ span_flags, uint64_t spans,
                                                        uint32_t* __restrict__ span_tickets,
                                                        uint32_t* __restrict__ mbits,
                                                        uint32_t* __restrict__ ctrl, int* __restrict__ status) {
    __shared__ float sm[kAccThreads / 64];
    __shared__ uint32_t s_cc[kAccThreads / 64];
    __shared__ uint32_t s_part[kFTile + 1];   // per-tensor maxima of a tile that spans tensors
    __shared__ uint32_t s_start[kFTile + 1];  // their first elements, relative to the tile
    const uint32_t t = blockIdx.x;
    const uint32_t info = g.segs ? g.ftile_info[t] : 0u;  // issued before the stream loads
    const uint64_t i4 = (uint64_t)t * (kFTile / 4) + threadIdx.x;
    const uint64_t el = i4 << 2;
    float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (el + 4 <= N) {
        // x is read once and err is not read again on most tiles: stream all
        // three accesses past the caches (measured ~10% faster on MI355X
        // than plain loads and stores; the store is store_stream's)
        f4 a = __builtin_nontemporal_load(reinterpret_cast<const f4*>(x) + i4);
        const f4 b = __builtin_nontemporal_load(reinterpret_cast<const f4*>(err) + i4);
        if (x_div != 1.0f) a = a / x_div;  // the workers' mean (server direction); IEEE divide
        const f4 r = a + b;
        store_stream(reinterpret_cast<f4*>(err) + i4, r);
        v[0] = r.x;
        v[1] = r.y;
        v[2] = r.z;
        v[3] = r.w;
    } else {
        for (int j = 0; j < 4; ++j) {
            if (el + j < N) {
                const float xj = x_div != 1.0f ? x[el + j] / x_div : x[el + j];
                v[j] = xj + err[el + j];
                err[el + j] = v[j];
            }
        }
    }
    if (!(info & kStraddle)) {
        const float m = wave_max(fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
        // the tile's candidate list (elements with |v| >= the tensor's bound)
        const float cb = cand_bound(hint[info], s);
        // a list is in no particular order: component j of every lane, lane by
        // lane, after components 0..j-1; positions come from the ballots
        uint32_t cm = 0, ctot = 0, cpos[4] = {0u, 0u, 0u, 0u};
        if (cb != INFINITY) {
#pragma unroll
            for (int j = 0; j < 4; ++j) cm |= (uint32_t)(fabsf(v[j]) >= cb) << j;
            if (__ballot(cm != 0)) {  // most waves have none
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint64_t b = __ballot((cm >> j) & 1);
                    cpos[j] = ctot + __builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32),
                                                               __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
                    ctot += (uint32_t)__popcll(b);
                }
            }
        }
        if (lane_id() == 0) {
            sm[wave_id()] = m;
            s_cc[wave_id()] = ctot;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            float r = sm[0];
#pragma unroll
            for (int k = 1; k < kAccThreads / 64; ++k) r = fmaxf(r, sm[k]);
            pmax[t + info] = r;
        }
        uint32_t before = 0, total = 0;
#pragma unroll
        for (int k = 0; k < kAccThreads / 64; ++k) {
            before += k < wave_id() ? s_cc[k] : 0u;
            total += s_cc[k];
        }
        if (cb != INFINITY && total <= kCand) {
            uint2* const lst = cand + (uint64_t)t * kCand + before;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if ((cm >> j) & 1) lst[cpos[j]] = make_uint2(4 * threadIdx.x + j, __float_as_uint(v[j]));
        }
        if (threadIdx.x == 0) cand_cnt[t] = (cb != INFINITY && total <= kCand) ? (uint16_t)total : kCandNone;
    } else {
        // the tile spans tensors g0..g1: one partial max per tensor, in slot
        // t + g.  The first elements of the tensors that can meet it (g0 up
        // to the tensor of the next tile's first element: at most kFTile + 1,
        // as no tensor is empty) go to LDS, where each element finds its
        // tensor without a search through the table.
        const uint32_t g0 = info & ~kStraddle;
        const uint64_t tile0 = (uint64_t)t * kFTile;
        const uint64_t last = min(N, tile0 + kFTile) - 1;
        const uint32_t gn = tile0 + kFTile < N ? (g.ftile_info[t + 1] & ~kStraddle) : g.count - 1;
        const uint32_t nk = gn - g0 + 1;
        for (uint32_t k = threadIdx.x; k < nk; k += kAccThreads) {
            const uint64_t eo = g.segs[g0 + k].elem_off;
            s_start[k] = eo <= tile0 ? 0u : (uint32_t)min<uint64_t>(eo - tile0, kFTile);
            s_part[k] = 0;
        }
        __syncthreads();
        auto tensor_of = [&](uint32_t i) {  // the last k with s_start[k] <= i (s_start[0] == 0)
            uint32_t lo = 0, hi = nk;
            while (hi - lo > 1) {
                const uint32_t mid = (lo + hi) >> 1;
                if (s_start[mid] <= i) lo = mid;
                else hi = mid;
            }
            return lo;
        };
        for (int j = 0; j < 4; ++j) {
            if (el + j < N)  // order of non-negative floats
                atomicMax(&s_part[tensor_of((uint32_t)(el + j - tile0))], __float_as_uint(fabsf(v[j])));
        }
        const uint32_t klast = tensor_of((uint32_t)(last - tile0));
        __syncthreads();
        for (uint32_t k = threadIdx.x; k <= klast; k += kAccThreads) pmax[t + g0 + k] = __uint_as_float(s_part[k]);
        if (threadIdx.x == 0) cand_cnt[t] = kCandNone;  // a tile shared by tensors is read again in full
    }
    // look-back state of k_emit starts empty on every call
    for (uint64_t i = (uint64_t)t * kAccThreads + threadIdx.x; i < spans; i += (uint64_t)gridDim.x * kAccThreads)
        span_flags[i] = 0;
    for (uint64_t i = (uint64_t)t * kAccThreads + threadIdx.x; i < g.count; i += (uint64_t)gridDim.x * kAccThreads) {
        span_tickets[i] = 0;
        mbits[i] = 0;  // M of tensor i, raised by k_tile_max
    }
    if (t == 0 && threadIdx.x == 0) {
        ctrl[1] = 0;  // listed encode tiles
        *status = TLC_OK;
    }
}

constexpr int kActPerThread = 4;  // encode tiles per thread in k_tile_activity

__device__ __forceinline__ uint32_t etile_owner(const GroupView& g, uint32_t e) { return g.etile_seg ? g.etile_seg[e] : 0u; }

// max over the flat-tile partial maxima under encode tile j of a tensor
__device__ __forceinline__ float etile_max(const float* pm, const Seg& sg, uint32_t j) {
    const uint64_t a = sg.elem_off + (uint64_t)j * kETile;
    const uint64_t b = sg.elem_off + min((uint64_t)sg.n, (uint64_t)(j + 1) * kETile) - 1;
    const uint64_t t0 = a / kFTile, t1 = b / kFTile;  // at most kETile / kFTile + 1 flat tiles
    float mx = 0.0f;
#pragma unroll
    for (uint64_t k = 0; k <= kETile / kFTile; ++k)
        if (t0 + k <= t1) mx = fmaxf(mx, pm[t0 + k]);
    return mx;
}

// One thread per encode tile of the group: the tile's maximum |x+err| from
// the flat-tile partial maxima under it, and every tensor's M as the max over
// its tiles.  Tiles of one tensor are contiguous, so a segmented max over the
// wave leaves one atomic per tensor and wave; M (zeroed by k_accum_max) is
// kept as float bits, whose unsigned order is that of non-negative floats.
__global__ __launch_bounds__(kThreads) void k_tile_max(GroupView g, uint32_t etiles, const float* __restrict__ pmax,
                                                       float* __restrict__ etmax, uint32_t* __restrict__ mbits,
                                                       const float* __restrict__ hint, float s,
                                                       float* __restrict__ seg_cb) {
    const uint32_t e = blockIdx.x * kThreads + threadIdx.x;
    const int lane = lane_id();
    const bool ok = e < etiles;
    const uint32_t gi = ok ? etile_owner(g, e) : 0xFFFFFFFFu;
    float mx = 0.0f;
    if (ok) {
        const Seg sg = load_seg(g, gi);
        mx = etile_max(pmax + gi, sg, e - sg.etile0);  // flat tile t of tensor gi: slot t + gi
        etmax[e] = mx;
        // the bound the first pass used for the tensor's candidate lists (the
        // hint is the caller's M buffer, rewritten only by k_tile_activity)
        if (e == sg.etile0) seg_cb[gi] = cand_bound(hint[gi], s);
    }
    for (int d = 1; d < 64; d <<= 1) {
        const float o = __shfl_up(mx, d, 64);
        const uint32_t og = __shfl_up(gi, d, 64);
        if (lane >= d && og == gi) mx = fmaxf(mx, o);
    }
    const uint32_t next = __shfl_down(gi, 1, 64);
    if (ok && (lane == 63 || next != gi)) atomicMax(mbits + gi, __float_as_uint(mx));
}

// Per encode tile: M*s and the exact selection threshold of its tensor (the
// thread of a tensor's first tile writes M to the caller's buffer, which held
// the hint until now); a tile whose maximum reaches the threshold can hold
// nonzero codes and is listed for k_quant_pack, with the flat tiles under it
// that reach it and whether the tensor's candidate lists are complete; any
// other tile holds only zero codes and is summarised here as a run of byte
// 121.
__global__ __launch_bounds__(kThreads) void k_tile_activity(GroupView g, uint32_t etiles, float s,
                                                            const float* __restrict__ pmax,
                                                            const float* __restrict__ etmax,
                                                            const uint32_t* __restrict__ mbits,
                                                            const float* __restrict__ seg_cb,
                                                            float* __restrict__ scales,
                                                            uint64_t* __restrict__ etile_agg,
                                                            PackJob* __restrict__ jobs, uint32_t* __restrict__ ctrl) {
    __shared__ uint32_t s_u[kWaves];
    __shared__ uint32_t s_base;
    const uint32_t base = blockIdx.x * (kThreads * kActPerThread);
    // the thread's tiles go through each dependent load step together
    uint32_t gis[kActPerThread];
#pragma unroll
    for (int r = 0; r < kActPerThread; ++r) {
        const uint32_t e = base + r * kThreads + threadIdx.x;
        gis[r] = e < etiles ? etile_owner(g, e) : 0u;
    }
    Seg sgs[kActPerThread];
    float ms_[kActPerThread], tmax[kActPerThread], cbs[kActPerThread];
#pragma unroll
    for (int r = 0; r < kActPerThread; ++r) {
        const uint32_t e = base + r * kThreads + threadIdx.x;
        sgs[r] = load_seg(g, gis[r]);
        ms_[r] = __uint_as_float(mbits[gis[r]]);
        cbs[r] = seg_cb[gis[r]];
        tmax[r] = e < etiles ? etmax[e] : 0.0f;
    }
    uint32_t mask = 0;
    PackJob jb[kActPerThread] = {};
#pragma unroll
    for (int r = 0; r < kActPerThread; ++r) {
        const uint32_t e = base + r * kThreads + threadIdx.x;
        if (e < etiles) {
            const Seg& sg = sgs[r];
            const float m = ms_[r];
            const float ms = m * s;
            const float thr = select_threshold(m, ms);
            const uint32_t j = e - sg.etile0;
            if (j == 0) scales[gis[r]] = m;  // the caller's M (it held the hint until now)
            if (tmax[r] >= thr) {
                mask |= 1u << r;
                jb[r].e0 = sg.elem_off + (uint64_t)j * kETile;
                jb[r].et = e;
                jb[r].nel = min(kETile, sg.n - j * kETile);
                jb[r].thr = thr;
                jb[r].ms = ms;
                jb[r].gi = gis[r];
            } else {
                const uint32_t B = quartic_len(sg.n);
                etile_agg[e] = carry_pack(carry_run(min(kETileBytes, B - j * kETileBytes)));
            }
        }
    }
    // which flat tiles under a listed tile reach the threshold: every load
    // is issued before the first compare
    constexpr int kSub = kETile / kFTile + 1;  // flat tiles an encode tile can touch
    float pv[kActPerThread][kSub];
#pragma unroll
    for (int r = 0; r < kActPerThread; ++r) {
        const bool act = (mask >> r) & 1;
        const uint64_t t0 = act ? jb[r].e0 / kFTile : 0, t1 = act ? (jb[r].e0 + jb[r].nel - 1) / kFTile : 0;
        const float* pm = pmax + (act ? jb[r].gi : 0u) + t0;  // flat tile t of tensor gi: slot t + gi
#pragma unroll
        for (int k = 0; k < kSub; ++k) {
            pv[r][k] = -1.0f;
            if (act && t0 + k <= t1) pv[r][k] = pm[k];
        }
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmem);
#pragma unroll
    for (int r = 0; r < kActPerThread; ++r) {
        uint32_t fm = 0;
#pragma unroll
        for (int k = 0; k < kSub; ++k) fm |= (uint32_t)(pv[r][k] >= jb[r].thr) << k;
        // every element with a nonzero code is on its flat tile's list when
        // the threshold is at least the bound the lists were cut at
        if (jb[r].thr >= cbs[r] && (jb[r].e0 & 3) == 0) fm |= kCandOk;
        jb[r].fmask = fm;
    }
    // compaction: one atomic per block
    uint32_t tot;
    const uint32_t before = block_excl_sum(__popc(mask), s_u, &tot);
    if (tot == 0) return;
    if (threadIdx.x == 0) s_base = atomicAdd(ctrl + 1, tot);
    __syncthreads();
    uint32_t pos = s_base + before;
#pragma unroll
    for (int r = 0; r < kActPerThread; ++r)
        if (mask & (1u << r)) jobs[pos++] = jb[r];
}

// LDS writes of one lane visible to the other lanes of its wave
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Per-wave LDS slice of k_quant_pack: the tile's codes (one int8 per element),
// its staged stream bytes, and a bitmap of its literal quartic bytes.
constexpr uint32_t kSliceStage = kETile;                      // offset of the staged bytes
constexpr uint32_t kSliceBits = kSliceStage + kETileBytes;    // offset of the bitmap
constexpr uint32_t kSlice = kSliceBits + kETileBytes / 8;     // bytes per wave

// Marks the quartic bytes of tile elements u..u+3 that hold a nonzero code
// (four elements touch at most two bytes).
__device__ __forceinline__ void mark_literals(uint32_t* lit, uint32_t u, int q0, int q1, int q2, int q3) {
    const uint32_t b0 = u / 5, split = 5 * (b0 + 1) - u;  // elements d < split lie in byte b0
    const bool f0 = q0 || (q1 && split > 1) || (q2 && split > 2) || (q3 && split > 3);
    const bool f1 = (q1 && split <= 1) || (q2 && split <= 2) || (q3 && split <= 3);
    if (f0) atomicOr(lit + (b0 >> 5), 1u << (b0 & 31));
    if (f1) atomicOr(lit + ((b0 + 1) >> 5), 1u << ((b0 + 1) & 31));
}

// One wavefront quantizes, packs and zero-run encodes one encode tile.  Only
// the flat tiles (512 elements) whose max reaches the threshold are read: from
// their candidate lists when the tensor's lists are complete (and the tile's
// did not overflow), else from err again.  Every other element has code 0 and
// err = v already, so it needs no HBM traffic.  The job comes in scalar
// registers, so the tile's first vector loads are its data.  Codes go to this wave's LDS slice, and every
// quartic byte that holds a nonzero code (a literal) is marked in a bitmap;
// the zero-run encoding then works literal by literal (64 per round), which
// costs nothing for the runs of byte 121 that make up most of a tile.
__device__ void pack_tile(const GroupView& g, const PackJob& jb, float* __restrict__ err,
                          uint64_t* __restrict__ etile_agg, uint8_t* __restrict__ staging,
                          const uint16_t* __restrict__ cand_cnt, const uint2* __restrict__ cand, const FixedOut& fo,
                          int8_t* slice) {
    const int lane = lane_id();
    const uint64_t e0 = jb.e0;
    const uint32_t et = jb.et, nel = jb.nel;
    const uint32_t nbytes = (nel + 4) / 5;
    const float thr = jb.thr, ms = jb.ms;
    int8_t* const q = slice;
    uint8_t* const stage = reinterpret_cast<uint8_t*>(slice + kSliceStage);
    uint32_t* const lit = reinterpret_cast<uint32_t*>(slice + kSliceBits);

    // every code starts at 0 (pad codes past the tensor end included), no
    // byte is marked, and the staged bytes start as 255 (a full 14-run), so
    // only remainder codes and literals are written there later
#pragma unroll
    for (int k = 0; k < kETile / 1024; ++k) reinterpret_cast<uint4*>(q)[lane + 64 * k] = make_uint4(0u, 0u, 0u, 0u);
    reinterpret_cast<uint4*>(stage)[lane] = make_uint4(~0u, ~0u, ~0u, ~0u);
    if (lane < 32) lit[lane] = 0u;

    const uint64_t ta0 = e0 / kFTile;
    uint32_t m = jb.fmask & ~kCandOk;  // active flat tiles still to be read in full
    if (jb.fmask & kCandOk) {
        // Flat tiles with a list: every element with a nonzero code is on it,
        // with its v, so only the list is read.  Lane f < 11 holds flat tile
        // ta0 + f; the lists are taken 4 x 64 candidates per round.
        const uint32_t nft = (uint32_t)((e0 + nel - 1) / kFTile - ta0) + 1;
        const bool act = (uint32_t)lane < nft && ((m >> lane) & 1);
        // The counts of flat tiles ta0 .. ta0 + 10 lie in 7 aligned words from
        // word ta0 / 2 (read past the last count stays inside the workspace).
        // The address is wave-uniform, so these are scalar loads, which do not
        // wait behind the vector stores of the wave's previous tile.
        const uint32_t* const cw = reinterpret_cast<const uint32_t*>(cand_cnt) + (ta0 >> 1);
        uint32_t cwords[7];
#pragma unroll
        for (int k = 0; k < 7; ++k) cwords[k] = cw[k];
        const uint32_t hw = (uint32_t)(ta0 & 1) + (uint32_t)lane;  // half-word holding flat tile ta0 + lane
        uint32_t wsel = 0;
#pragma unroll
        for (int k = 0; k < 7; ++k) wsel = (hw >> 1) == (uint32_t)k ? cwords[k] : wsel;
        const uint32_t c = act ? ((hw & 1) ? wsel >> 16 : wsel & 0xFFFFu) : 0u;
        const uint32_t ovf = (uint32_t)__ballot(act && c == kCandNone);
        uint32_t C;
        const uint32_t pre = wave_excl_sum(act && c != kCandNone ? c : 0u, &C);
        uint32_t pres[kETile / kFTile + 1];  // first candidate number of each flat tile
#pragma unroll
        for (int f = 0; f <= (int)(kETile / kFTile); ++f) pres[f] = __shfl(pre, f, 64);
        for (uint32_t base = 0; base < C; base += 4 * 64) {
            uint64_t at[4];
            uint32_t idx[4];
            float val[4];
            bool ok[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t k = base + 64 * r + lane;
                ok[r] = k < C;
                int f = 0;      // last flat tile whose first candidate number is <= k
                uint32_t pf = 0;
#pragma unroll
                for (int j = 1; j <= (int)(kETile / kFTile); ++j) {
                    const bool le = pres[j] <= k && (uint32_t)j < nft;
                    f = le ? j : f;
                    pf = le ? pres[j] : pf;
                }
                at[r] = (ta0 + f) * kCand + (k - pf);
                idx[r] = 0;
                val[r] = 0.0f;
                if (ok[r]) {
                    const uint2 c2 = cand[at[r]];
                    idx[r] = c2.x;
                    val[r] = __uint_as_float(c2.y);
                }
                at[r] = (ta0 + f) * kFTile;  // the flat tile's first element
            }
            __builtin_amdgcn_s_waitcnt(kWaitVmem);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t u = (int64_t)(at[r] + idx[r]) - (int64_t)e0;  // tile element
                if (ok[r] && u >= 0 && u < (int64_t)nel) {
                    const int qq = ternary(val[r], thr);
                    if (qq) {
                        err[e0 + u] = val[r] - (float)qq * ms;
                        q[u] = (int8_t)qq;
                        atomicOr(lit + (((uint32_t)u / 5) >> 5), 1u << (((uint32_t)u / 5) & 31));
                    }
                }
            }
        }
        m = ovf;
    }
    if ((e0 & 3) == 0) {
        // Active flat tiles, kPackSlots / 2 at a time.  A batch issues all its loads
        // (each one predicated, no branch writes a register another branch
        // loads into), waits for them once, and only then computes and
        // writes: so no wait inside the tile can fall on a store.  Four
        // consecutive elements never straddle two encode tiles here; only
        // the last float4 of a tensor whose size is not a multiple of 4 is
        // partial.
        uint32_t* const q4 = reinterpret_cast<uint32_t*>(q);
        while (m) {
            int64_t u[kPackSlots];
            bool full[kPackSlots], part[kPackSlots];
#pragma unroll
            for (int h = 0; h < kPackSlots / 2; ++h) {
                const int f = m ? __builtin_ctz(m) : -1;
                if (m) m &= m - 1;
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    const int slot = 2 * h + k;
                    u[slot] = f < 0 ? -1 : (int64_t)((ta0 + f) * kFTile) - (int64_t)e0 + 4 * lane + 256 * k;
                    full[slot] = u[slot] >= 0 && u[slot] + 4 <= (int64_t)nel;
                    part[slot] = u[slot] >= 0 && u[slot] < (int64_t)nel && !full[slot];
                }
            }
            f4 v[kPackSlots];
            float p0[kPackSlots], p1[kPackSlots], p2[kPackSlots];
#pragma unroll
            for (int slot = 0; slot < kPackSlots; ++slot) {
                v[slot] = f4{0.0f, 0.0f, 0.0f, 0.0f};
                p0[slot] = p1[slot] = p2[slot] = 0.0f;
                const float* const a = err + e0 + u[slot];
                if (full[slot]) v[slot] = *reinterpret_cast<const f4*>(a);
                if (part[slot]) {
                    p0[slot] = a[0];
                    if (u[slot] + 1 < (int64_t)nel) p1[slot] = a[1];
                    if (u[slot] + 2 < (int64_t)nel) p2[slot] = a[2];
                }
            }
            __builtin_amdgcn_s_waitcnt(kWaitVmem);
            f4 nv[kPackSlots];
            int qs[kPackSlots][4];
#pragma unroll
            for (int slot = 0; slot < kPackSlots; ++slot) {
                if (part[slot]) v[slot] = f4{p0[slot], p1[slot], p2[slot], 0.0f};
                qs[slot][0] = ternary(v[slot].x, thr);
                qs[slot][1] = ternary(v[slot].y, thr);
                qs[slot][2] = ternary(v[slot].z, thr);
                qs[slot][3] = ternary(v[slot].w, thr);  // 0 past the tensor end (v = 0)
                nv[slot] = f4{v[slot].x - (float)qs[slot][0] * ms, v[slot].y - (float)qs[slot][1] * ms,
                              v[slot].z - (float)qs[slot][2] * ms, v[slot].w - (float)qs[slot][3] * ms};
                if (full[slot] || part[slot]) {
                    q4[u[slot] >> 2] = (uint32_t)(uint8_t)(int8_t)qs[slot][0] |
                                       (uint32_t)(uint8_t)(int8_t)qs[slot][1] << 8 |
                                       (uint32_t)(uint8_t)(int8_t)qs[slot][2] << 16 |
                                       (uint32_t)(uint8_t)(int8_t)qs[slot][3] << 24;
                    mark_literals(lit, (uint32_t)u[slot], qs[slot][0], qs[slot][1], qs[slot][2], qs[slot][3]);
                }
            }
            // only the elements with a nonzero code change (err = v already
            // holds for the others): partial writes cost less HBM time than
            // writing the flat tiles back whole once most tiles are active
#pragma unroll
            for (int slot = 0; slot < kPackSlots; ++slot) {
                float* const a = err + e0 + u[slot];
                if (full[slot] || part[slot]) {
                    if (qs[slot][0]) a[0] = nv[slot].x;
                    if (qs[slot][1]) a[1] = nv[slot].y;
                    if (qs[slot][2]) a[2] = nv[slot].z;
                    if (qs[slot][3]) a[3] = nv[slot].w;  // 0 for a partial float4
                }
            }
        }
    } else {
        // a tensor that starts off a 16-byte boundary: element by element
        for (uint32_t u = lane; u < nel; u += 64) {
            if ((m >> ((e0 + u) / kFTile - ta0)) & 1) {
                const float vv = err[e0 + u];
                const int qq = ternary(vv, thr);
                if (qq) {
                    err[e0 + u] = vv - (float)qq * ms;
                    atomicOr(lit + ((u / 5) >> 5), 1u << ((u / 5) & 31));
                }
                q[u] = (int8_t)qq;
            }
        }
    }
    wave_sync();

    if (fo.enc) {
        // fixed-length encodings: lane l packs codes 80l..80l+79 (20 words of
        // LDS) into its 16 quartic bytes or 20 two-bit bytes at a fixed place
        const Seg sg = load_seg(g, jb.gi);
        const uint32_t TB = fixed_tile_bytes(fo.enc);
        const uint64_t j = et - sg.etile0;
        const uint32_t nb = (uint32_t)min((uint64_t)TB, fixed_len_of(sg.n, fo.enc) - j * TB);
        uint8_t* const dst = fo.out + (fo.offs ? fo.offs[jb.gi] : 0ull) + j * TB;
        uint32_t words[20];
#pragma unroll
        for (int i = 0; i < 20; ++i) words[i] = reinterpret_cast<const uint32_t*>(q)[20 * lane + i];
        uint32_t ob[5];  // up to 20 output bytes, 4 per word
        uint32_t nout;
        if (fo.enc == TLC_ENC_QUARTIC) {
            nout = 16;
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                uint32_t word = 0;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    uint32_t byte = 0, w3 = 1;
#pragma unroll
                    for (int d = 0; d < 5; ++d) {
                        const int idx = 20 * gq + 5 * jj + d;
                        const int qq = (int)(int8_t)(words[idx >> 2] >> (8 * (idx & 3)));
                        byte += (uint32_t)(qq + 1) * w3;
                        w3 *= 3;
                    }
                    word |= byte << (8 * jj);
                }
                ob[gq] = word;
            }
            ob[4] = 0;
        } else {
            nout = 20;
#pragma unroll
            for (int b = 0; b < 20; ++b) {
                uint32_t byte = 0;
#pragma unroll
                for (int d = 0; d < 4; ++d) byte |= ((((words[b] >> (8 * d)) & 0xFFu) + 1u) & 3u) << (2 * d);
                if ((b & 3) == 0) ob[b >> 2] = 0;
                ob[b >> 2] |= byte << (8 * (b & 3));
            }
        }
        const uint32_t o0 = nout * lane;
        if (o0 + nout <= nb && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
            if (nout == 16) {
                *reinterpret_cast<uint4*>(dst + o0) = make_uint4(ob[0], ob[1], ob[2], ob[3]);
            } else {
#pragma unroll
                for (int k = 0; k < 5; ++k) reinterpret_cast<uint32_t*>(dst + o0)[k] = ob[k];
            }
        } else {
            for (uint32_t b = 0; b < nout; ++b)
                if (o0 + b < nb) dst[o0 + b] = (uint8_t)(ob[b >> 2] >> (8 * (b & 3)));
        }
        wave_sync();  // the LDS slice is rewritten by the wave's next tile
        return;
    }

    // Literal n of the tile (in byte order) is found by rank: lanes 0..31
    // hold the bitmap words, a prefix sum of their popcounts gives each
    // word's first rank.  Each literal emits, after the previous literal at
    // distance g + 1: g / 14 bytes 255, the remainder code of g mod 14 (if
    // not 0) and itself; the first literal emits only itself (the run before
    // it is part of the carry summary).
    const uint32_t w = lane < 32 ? lit[lane] : 0u;
    uint32_t L;
    const uint32_t wpre = wave_excl_sum((uint32_t)__popc(w), &L);
    Carry agg = carry_run(nbytes);
    uint32_t k_int = 0;
    if (L) {
        uint32_t out_base = 0;  // staged bytes of earlier rounds
        int prev_last = 0, first = 0;
        for (uint32_t c0 = 0; c0 < L; c0 += 64) {
            const uint32_t n = c0 + lane;
            const bool has = n < L;
            int wi = 0;  // last bitmap word whose first rank is <= n
#pragma unroll
            for (int step = 16; step >= 1; step >>= 1) {
                const uint32_t pc = __shfl(wpre, wi + step, 64);
                if (pc <= n) wi += step;
            }
            uint32_t x = __shfl(w, wi, 64);
            uint32_t r = n - __shfl(wpre, wi, 64);  // rank inside the word
            int pos = 0;
#pragma unroll
            for (int step = 16; step >= 1; step >>= 1) {
                const uint32_t c = (uint32_t)__popc(x & ((1u << step) - 1u));
                if (r >= c) {
                    r -= c;
                    x >>= step;
                    pos += step;
                }
            }
            const int k = has ? 32 * wi + pos : 0;  // quartic byte index of literal n
            uint32_t val = 0;
            if (has) {
                uint32_t w3 = 1;
#pragma unroll
                for (int d = 0; d < 5; ++d) {
                    val += (uint32_t)((int)q[5 * k + d] + 1) * w3;
                    w3 *= 3;
                }
            }
            int pk = __shfl_up(k, 1, 64);
            if (lane == 0) pk = prev_last;
            const uint32_t g = (uint32_t)(k - pk - 1);
            const uint32_t len = !has ? 0u : (n == 0 ? 1u : g / kRunMax + (g % kRunMax != 0) + 1u);
            uint32_t tot;
            const uint32_t ex = wave_excl_sum(len, &tot);
            if (has) {
                const uint32_t end = out_base + ex + len;  // one past this literal's bytes
                stage[end - 1] = (uint8_t)val;
                if (n != 0 && g % kRunMax) stage[end - 2] = remainder_code(g % kRunMax);
            }
            out_base += tot;
            if (c0 == 0) first = __shfl(k, 0, 64);
            prev_last = __shfl(k, (int)min(64u, L - c0) - 1, 64);
        }
        const uint32_t t = nbytes - 1 - (uint32_t)prev_last;  // zero bytes after the last literal
        k_int = out_base + t / kRunMax;                       // their full runs stay 255
        wave_sync();
        if (16u * lane < k_int)
            reinterpret_cast<uint4*>(staging + (uint64_t)et * kETileBytes)[lane] =
                reinterpret_cast<const uint4*>(stage)[lane];
        agg.lit = 1;
        agg.p = (uint32_t)first % kRunMax;
        agg.K = (uint32_t)first / kRunMax + k_int;
        agg.c = t % kRunMax;
    }
    if (lane == 0) etile_agg[et] = carry_pack(agg) | ((uint64_t)k_int << 32);
    wave_sync();  // the LDS slice is rewritten by the wave's next tile
}

__global__ __launch_bounds__(kThreads) void k_quant_pack(GroupView g, float* __restrict__ err,
                                                         const PackJob* __restrict__ jobs,
                                                         const uint32_t* __restrict__ ctrl,
                                                         uint64_t* __restrict__ etile_agg,
                                                         uint8_t* __restrict__ staging,
                                                         const uint16_t* __restrict__ cand_cnt,
                                                         const uint2* __restrict__ cand, FixedOut fo) {
    __shared__ __align__(16) int8_t s_q[kWaves * kSlice];
    const uint32_t na = ctrl[1];
    const uint32_t wave = __builtin_amdgcn_readfirstlane(wave_id());
    const uint32_t waves = gridDim.x * kWaves;
    for (uint32_t i = blockIdx.x * kWaves + wave; i < na; i += waves)
        pack_tile(g, jobs[i], err, etile_agg, staging, cand_cnt, cand, fo, s_q + wave * kSlice);
}

// Bytes of a span's output that k_emit assembles in LDS at a time (an
// all-zero span of 256 encode tiles needs ~18.7 KB, a span of the BERT-large
// set after many error-feedback steps ~35-45 KB); a larger output goes out in
// several windows.  With the block's other arrays this keeps three blocks per
// CU (160 KB of LDS), so the ~560 spans of a 340M-value set are resident at
// once.
constexpr uint32_t kEmitLds = 40960;

// Staged chunks of a span up to which k_emit keeps a table of each chunk's
// tile in LDS (one byte each) instead of searching the tiles' chunk prefix
// for every chunk: a span of the BERT-large set holds ~1,200-2,600.
constexpr uint32_t kOwnCap = 4096;

__device__ __forceinline__ uint8_t byte_of(const uint4& v, uint32_t i) {  // byte i (0..15) of v
    const uint32_t w = i < 4 ? v.x : i < 8 ? v.y : i < 12 ? v.z : v.w;
    return (uint8_t)(w >> (8 * (i & 3)));
}

// One block per span of 256 encode tiles of a tensor: block scan of the
// tiles' carry summaries, decoupled look-back across the tensor's spans for
// the span's input state, then the span's stream bytes.
__global__ __launch_bounds__(kThreads) void k_emit(GroupView g, const uint64_t* __restrict__ etile_agg,
                                                   const uint8_t* __restrict__ staging,
                                                   uint64_t* __restrict__ flags, uint32_t* __restrict__ tickets,
                                                   uint8_t* __restrict__ out, uint64_t* __restrict__ out_lens,
                                                   int* __restrict__ status) {
    __shared__ uint64_t s_sm[kWaves];
    __shared__ uint32_t s_u[kWaves];
    __shared__ uint32_t s_off[kThreads + 1];  // output offset of each tile within the span
    __shared__ uint32_t s_dst[kThreads];      // stream position of each tile's first byte
    __shared__ uint32_t s_lead[kThreads];     // 255 codes that open the tile's output
    __shared__ uint16_t s_kint[kThreads];     // staged bytes after the lead (and remainder code)
    __shared__ uint8_t s_rem[kThreads];       // remainder code after the 255s, or 0
    __shared__ uint8_t s_fin[kThreads];       // closing remainder code of the tensor's last tile, or 0
    __shared__ uint32_t s_cpre[kThreads + 1];  // prefix of staged 16-byte chunks over the span's tiles
    __shared__ __align__(16) uint32_t s_out[(kEmitLds + 16) / 4];  // the span's bytes, inverted and shifted by the store misalignment
    __shared__ uint8_t s_own[kOwnCap];           // tile of each staged chunk (spans of at most kOwnCap chunks)
    __shared__ uint32_t s_span, s_E, s_r, s_ok, s_clo, s_chi;

    // Block b belongs to the tensor of span b.  A tensor with several spans
    // hands them out in ticket order from its own counter, so that the
    // look-back only ever waits for blocks that already hold a smaller
    // ticket; a single-span tensor needs no ticket.
    const uint32_t ent = g.segs ? g.span_seg[blockIdx.x] : (etiles_of(g.one.n) > kSpan ? kMulti : 0u);
    const uint32_t gi = ent & ~kMulti;
    if (threadIdx.x == 0) s_span = (ent & kMulti) ? atomicAdd(tickets + gi, 1u) : 0u;  // in flight with the record
    const Seg sg = load_seg(g, gi);
    const uint32_t B = quartic_len(sg.n), ne = etiles_of(sg.n);
    __syncthreads();
    const uint32_t lsp = s_span;
    const uint32_t sp = sg.span0 + lsp;
    const uint32_t j = lsp * kSpan + threadIdx.x;  // tensor-relative encode tile
    const bool valid = j < ne;
    const uint32_t nb = valid ? min(kETileBytes, B - j * kETileBytes) : 0u;
    const uint64_t word = valid ? etile_agg[sg.etile0 + j] : 0ull;
    const Carry a = carry_unpack(word);
    uint32_t kint = (uint32_t)(word >> 32) & 0x7FFu;
    if (!a.lit) kint = 0;
    uint64_t total;
    const uint64_t excl = block_excl_scan(carry_pack(a), 0ull, CarryCompose(), s_sm, &total);

    // The staged bytes of the span's tiles do not depend on the look-back:
    // they move in aligned 16-byte chunks (chunk c of a tile holds its staged
    // bytes 16c .. 16c + 15), and the first 256 chunks are loaded before it.
    const uint8_t* const stg = staging + (uint64_t)(sg.etile0 + lsp * kSpan) * kETileBytes;
    uint32_t tot_chunks;
    const uint32_t my_chunks = (kint + 15) / 16;
    const uint32_t my_first = block_excl_sum(my_chunks, s_u, &tot_chunks);
    s_cpre[threadIdx.x] = my_first;
    if (threadIdx.x == 0) s_cpre[kThreads] = tot_chunks;
    const bool own = tot_chunks <= kOwnCap;  // block-uniform
    if (own)
        for (uint32_t i = 0; i < my_chunks; ++i) s_own[my_first + i] = (uint8_t)threadIdx.x;
    __syncthreads();
    auto chunk_owner = [&](uint32_t cv) -> uint32_t {  // tile holding staged chunk cv of the span
        if (own) return s_own[cv];
        uint32_t k = 0, hi2 = kThreads;
        while (hi2 - k > 1) {
            const uint32_t mid = (k + hi2) >> 1;
            if (s_cpre[mid] <= cv) k = mid;
            else hi2 = mid;
        }
        return k;
    };
    auto load_chunk = [&](uint32_t k, uint32_t cv) {
        return reinterpret_cast<const uint4*>(stg + (uint64_t)k * kETileBytes)[cv - s_cpre[k]];
    };
    uint32_t k0 = 0, v0x = 0, v0y = 0, v0z = 0, v0w = 0;  // (held in registers across the look-back)
    if (threadIdx.x < tot_chunks) {
        k0 = chunk_owner(threadIdx.x);
        const uint4 c = load_chunk(k0, threadIdx.x);
        v0x = c.x;
        v0y = c.y;
        v0z = c.z;
        v0w = c.w;
    }

    if (threadIdx.x < 64) {
        uint32_t E = 0, r = 0, ok = 1;
        if (lsp == 0) {
            if (threadIdx.x == 0) {
                uint32_t E2, r2;
                carry_apply(carry_unpack(total), 0, 0, &E2, &r2);
                publish(flags, sp, kPrefix, (uint64_t)E2 | ((uint64_t)r2 << 57));
            }
        } else {
            if (threadIdx.x == 0) publish(flags, sp, kAggregate, total);
            uint64_t f = 0;
            ok = look_back(flags, sp, sg.span0, 0ull, CarryCompose(), &f) ? 1u : 0u;
            if (ok) carry_apply(carry_unpack(f), 0, 0, &E, &r);
            if (threadIdx.x == 0) {
                if (ok) {
                    uint32_t E2, r2;
                    carry_apply(carry_unpack(total), E, r, &E2, &r2);
                    publish(flags, sp, kPrefix, (uint64_t)E2 | ((uint64_t)r2 << 57));
                } else {
                    publish(flags, sp, kPoison, 0);
                }
            }
        }
        if (threadIdx.x == 0) {
            s_E = E;
            s_r = r;
            s_ok = ok;
        }
    }
    __syncthreads();
    if (!s_ok) {
        if (threadIdx.x == 0) raise_status(status, TLC_ERR_INTERNAL);
        return;
    }

    uint32_t E_in, r_in;
    carry_apply(carry_unpack(excl), s_E, s_r, &E_in, &r_in);
    uint32_t lead = 0, rem = 0, fin = 0, len = 0;
    if (valid) {
        uint32_t E_out, r_out;
        if (!a.lit) {
            const uint32_t t = r_in + nb;
            lead = t / kRunMax;
            E_out = E_in + lead;
            r_out = t % kRunMax;
        } else {
            const uint32_t f = kRunMax * (a.K - kint) + a.p;  // first literal of the tile
            const uint32_t t = r_in + f;
            lead = t / kRunMax;
            rem = (t % kRunMax) ? remainder_code(t % kRunMax) : 0u;
            E_out = E_in + lead + (rem ? 1u : 0u) + kint;
            r_out = a.c;
        }
        len = E_out - E_in;
        if (j == ne - 1) {
            if (r_out) {
                fin = remainder_code(r_out);
                len += 1;
            }
            const uint64_t L = (uint64_t)E_out + (r_out ? 1u : 0u);
            if (L > B) raise_status(status, TLC_ERR_INTERNAL);
            out_lens[gi] = L;
        }
    }
    s_dst[threadIdx.x] = E_in;
    s_lead[threadIdx.x] = lead;
    s_kint[threadIdx.x] = (uint16_t)kint;
    s_rem[threadIdx.x] = (uint8_t)rem;
    s_fin[threadIdx.x] = (uint8_t)fin;
    uint32_t tot_len;
    s_off[threadIdx.x] = block_excl_sum(len, s_u, &tot_len);
    if (threadIdx.x == 0) s_off[kThreads] = tot_len;
    __syncthreads();

    // The span's tiles are consecutive in one tensor, so its output is the
    // contiguous stream range [D, D + tot_len), D = stream position of tile 0:
    // byte 255 except for each tile's remainder code after its leading 255s,
    // its staged bytes, and the tensor's closing remainder code.
    const uint32_t D = s_dst[0];
    const uint32_t end = min(tot_len, B - min(B, D));  // never past the tensor's slot
    uint8_t* const o = out + sg.stream_off + D;
    const uint32_t mis = (uint32_t)(reinterpret_cast<uintptr_t>(o) & 15);
    const uint32_t nchunks = end ? (mis + end + 15) / 16 : 0u;
    // Staged chunks cv_lo .. cv_hi - 1 of the span, 4 per thread and round
    // with every load issued before the first byte is placed (chunk t was
    // loaded by thread t before the look-back); put(p, nb, v) places the
    // first nb bytes of v (nb >= 1) at span bytes p .. p + nb - 1.
    auto copy_staged = [&](uint32_t cv_lo, uint32_t cv_hi, auto put) {
        for (uint32_t base = cv_lo; base < cv_hi; base += 4 * kThreads) {
            uint32_t kk[4];
            uint4 val[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t cv = base + r * kThreads + threadIdx.x;
                kk[r] = 0;
                val[r] = make_uint4(0u, 0u, 0u, 0u);
                if (cv < cv_hi) {
                    kk[r] = cv == threadIdx.x ? k0 : chunk_owner(cv);
                    val[r] = cv == threadIdx.x ? make_uint4(v0x, v0y, v0z, v0w) : load_chunk(kk[r], cv);
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t cv = base + r * kThreads + threadIdx.x;
                if (cv < cv_hi) {
                    const uint32_t k = kk[r];
                    const uint32_t c16 = 16 * (cv - s_cpre[k]);  // first staged byte of the chunk
                    const uint32_t sbase = s_off[k] + s_lead[k] + (s_rem[k] ? 1u : 0u) + c16;
                    if (sbase < end) put(sbase, min(min(16u, (uint32_t)s_kint[k] - c16), end - sbase), val[r]);
                }
            }
        }
    };

    // The output goes out in windows of kEmitLds bytes (one window for all
    // but the densest spans).  A window is assembled in LDS, where span byte
    // p is byte p - lo of s_out (lo: the span byte of the window's first
    // aligned 16-byte store chunk) and holds the stream byte inverted: the
    // buffer starts at zero (all bytes 255) and every exception byte is OR-ed
    // in, so neighbouring tiles' bytes that share a word need no ordering.
    // Then one aligned 16-byte store per chunk, inverted back: every stream
    // byte is written once and no barrier waits on HBM.
    constexpr uint32_t kWin = kEmitLds / 16;  // store chunks per window
    const uint32_t so = s_off[threadIdx.x] + lead + (rem ? 1u : 0u);  // span byte of this tile's first staged byte
    const bool one_window = nchunks <= kWin;  // block-uniform: the whole span in one window
    for (uint32_t w0 = 0; w0 < nchunks; w0 += kWin) {
        const uint32_t wn = min(kWin, nchunks - w0);
        const int32_t lo = (int32_t)(16 * w0) - (int32_t)mis;
        const int32_t hi = lo + (int32_t)(16 * wn);
        if (threadIdx.x == 0) {
            s_clo = ~0u;
            s_chi = 0u;
        }
        for (uint32_t c = threadIdx.x; c < wn; c += kThreads)
            reinterpret_cast<uint4*>(s_out)[c] = make_uint4(0u, 0u, 0u, 0u);
        __syncthreads();
        // the staged chunks that meet the window are consecutive: their range
        // is the min and max over the tiles (all of them when one window
        // holds the span), reduced per wavefront before the LDS atomics
        if (!one_window) {
            uint32_t clo = ~0u, chi = 0u;
            if (kint) {
                const int32_t a = max(lo - (int32_t)so, 0), b = min(hi - (int32_t)so, (int32_t)kint);
                if (a < b) {
                    clo = my_first + (uint32_t)a / 16;
                    chi = my_first + ((uint32_t)b + 15) / 16;
                }
            }
            for (int d = 32; d >= 1; d >>= 1) {
                clo = min(clo, (uint32_t)__shfl_xor((int)clo, d, 64));
                chi = max(chi, (uint32_t)__shfl_xor((int)chi, d, 64));
            }
            if (lane_id() == 0) {
                atomicMin(&s_clo, clo);
                atomicMax(&s_chi, chi);
            }
        }
        auto or_byte = [&](int32_t p, uint32_t b) {  // span byte p in [lo, hi)
            const uint32_t pos = (uint32_t)(p - lo);
            atomicOr(s_out + (pos >> 2), (~b & 0xFFu) << (8 * (pos & 3)));
        };
        {
            const int32_t pr = (int32_t)(s_off[threadIdx.x] + lead), pf = (int32_t)(s_off[threadIdx.x] + len) - 1;
            if (rem && pr < (int32_t)end && pr >= lo && pr < hi) or_byte(pr, rem);
            if (fin && pf < (int32_t)end && pf >= lo && pf < hi) or_byte(pf, fin);
        }
        if (!one_window) __syncthreads();  // s_clo, s_chi
        copy_staged(one_window ? 0u : s_clo, one_window ? tot_chunks : s_chi, [&](uint32_t p, uint32_t nb, uint4 v) {
            // bytes j of the chunk with j < nb and lo <= p + j < hi, inverted
            // (the others zeroed), shifted to the byte offset of p - lo in its
            // word, into the five words of s_out they meet
            const int32_t dst = (int32_t)p - lo;
            const int32_t jlo = max(-dst, 0), jhi = min((int32_t)nb, (int32_t)(16 * wn) - dst);
            auto inv = [&](uint32_t w, int32_t b0) {  // chunk bytes b0 .. b0 + 3
                const int32_t x = max(jlo - b0, 0), y = min(jhi - b0, 4);
                const uint32_t keep = y <= x ? 0u
                                             : (uint32_t)((((uint64_t)1 << (8 * (y - x))) - 1u) << (8 * x));
                return ~w & keep;
            };
            const uint32_t i0 = inv(v.x, 0), i1 = inv(v.y, 4), i2 = inv(v.z, 8), i3 = inv(v.w, 12);
            const uint32_t m = (uint32_t)dst & 3u;
            const int32_t wb = (dst - (int32_t)m) / 4;  // word of s_out holding byte dst (may be -1..-4)
            auto put_word = [&](int32_t i, uint32_t cur, uint32_t prev) {
                const uint32_t o = m == 0 ? cur : __builtin_amdgcn_alignbyte(cur, prev, 4u - m);
                if (o) atomicOr(s_out + (wb + i), o);  // o != 0 only for a word inside the window
            };
            put_word(0, i0, 0u);
            put_word(1, i1, i0);
            put_word(2, i2, i1);
            put_word(3, i3, i2);
            put_word(4, 0u, i3);
        });
        __syncthreads();
        for (uint32_t c = threadIdx.x; c < wn; c += kThreads) {
            const int64_t p0 = (int64_t)(w0 + c) * 16 - mis;  // span byte of the chunk's first byte
            uint8_t* const dst = o + p0;
            uint4 v = reinterpret_cast<const uint4*>(s_out)[c];
            v = make_uint4(~v.x, ~v.y, ~v.z, ~v.w);
            if (p0 >= 0 && p0 + 16 <= (int64_t)end) {
                *reinterpret_cast<uint4*>(dst) = v;
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (p0 + i >= 0 && p0 + i < (int64_t)end) dst[i] = byte_of(v, (uint32_t)i);
            }
        }
        __syncthreads();  // s_out is cleared for the next window
    }
}

// ---------------------------------------------------------------------------
// decompress kernels
//
// Decompress takes one of two launch sequences, both giving the same y:
// sparse streams (few encode tiles with a nonzero code): k_prep zero-fills y
// and k_decode writes the nonzero codes over the fill; dense streams:
// k_decode records where every encode tile begins and k_expand decodes each
// tile in LDS and writes it once.  The accumulate of one payload adds its
// nonzero codes to acc straight from the stream.  The accumulate of many
// payloads records the tile starts of every payload in one k_decode launch,
// then k_apply reads and writes each tile of acc once, decoding every
// payload's bytes for the tile in LDS and adding them in payload order.

// Where k_decode found encode tile j of a tensor to begin (decompress only):
// the stream byte, counted from the tensor's first, whose expansion holds
// quartic byte 1024 j, and how many quartic bytes of that expansion come
// before it (a run byte can straddle two tiles).
constexpr uint64_t kNoStart = ~0ull;

// k_decode's unit range bound meaning "through the last unit".
constexpr uint32_t kToEnd = ~0u;
__device__ __forceinline__ uint64_t tile_start(uint64_t byte, uint64_t skip) { return byte | skip << 32; }

// Stream density (bytes per quartic byte) above which the dense decompress
// path is faster: 104/1000, measured on MI355X over error-feedback runs of
// the BERT-large set, as the time of whole compress+decompress steps with
// each path forced (sparse ahead by 24 us at 0.094, dense ahead by 13 us at
// 0.109).  An all-zero stream holds 1/14 = 0.071 (runs of 14).
constexpr uint64_t kDenseNum = 104, kDenseDen = 1000;
// The same for the accumulate of many payloads (one pass over acc for all of
// them against one add pass per payload): 82/1000, measured on MI355X with 8
// BERT-large workers' payloads from 40 to 100 steps of error feedback (the
// add passes ahead by 116 us at 0.080, even at 0.082, behind by 73 us at
// 0.086).
constexpr uint64_t kManyDenseNum = 82;

constexpr uint32_t kMaxPayloads = 64;  // payloads of one accumulate-many call (one wavefront lane each)

// p[0 .. n) = v by one thread: 16-byte stores between a 4-byte head and tail.
__device__ __forceinline__ void fill_words(uint32_t* p, uint32_t n, uint32_t v) {
    uint32_t i = 0;
    for (; i < n && (reinterpret_cast<uintptr_t>(p + i) & 15); ++i) p[i] = v;
    const uint4 v4 = make_uint4(v, v, v, v);
    for (; i + 4 <= n; i += 4) *reinterpret_cast<uint4*>(p + i) = v4;
    for (; i < n; ++i) p[i] = v;
}

// Decoder state reset and set-up, for `payloads` payloads of the group (unit
// u = p * count + t is tensor t of payload p; in_lens and scales are indexed
// by unit).
// Sparse decompress (n_fill > 0): zero fill of y, one 16-byte store per lane
// (the fastest fill measured on MI355X; any load before the store, or more
// stores per lane, slows it by 10-40%), with store_stream: y is not read
// again here, and the kernels that follow (the caller's next compress) run
// faster when the caches do not hold y's dirty lines.  Dense decompress
// and accumulate-many (tstart set): the tile starts and literal flags of
// every payload are reset.
// Always: the look-back flags, and the list of stream chunks: unit u has
// max(1, ceil(min(L_u, B_t) / chunk)) chunks, numbered dec_first[u] ...;
// chunk r belongs to unit dec_map[r]; ctrl[3] = number of chunks.  Block 0
// also writes the density of the streams to *hint (when set): 1 if dense.
template <bool kFill>
__global__ __launch_bounds__(kThreads) void k_prep(GroupView g, uint32_t payloads, float* __restrict__ y,
                                                   uint64_t n_fill, const uint64_t* __restrict__ in_lens,
                                                   uint64_t* __restrict__ flags, uint64_t nflags,
                                                   uint64_t* __restrict__ tstart, uint32_t* __restrict__ tlit,
                                                   uint64_t ntiles, uint32_t* __restrict__ dec_map,
                                                   uint32_t* __restrict__ dec_first,
                                                   uint32_t* __restrict__ tickets, uint32_t* __restrict__ ctrl,
                                                   int* __restrict__ status, uint32_t* hint, uint32_t chunk,
                                                   uint32_t dense_num) {
    __shared__ uint32_t s_u[kWaves];
    __shared__ uint64_t s_d[2][kWaves];
    const uint64_t stride = (uint64_t)gridDim.x * kThreads;
    const uint64_t tid = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
    if (kFill) {  // a distinct kernel, so that profiles tell the two apart
        const uint64_t n4 = n_fill >> 2;
        float4* const y4 = reinterpret_cast<float4*>(y);
        for (uint64_t i = tid; i < n4; i += stride)
            store_stream(reinterpret_cast<f4*>(y4 + i), f4{0.0f, 0.0f, 0.0f, 0.0f});
        if (tid < (n_fill & 3)) y[(n4 << 2) + tid] = 0.0f;
    }
    for (uint64_t i = tid; i < nflags; i += stride) flags[i] = 0;
    if (tstart)
        for (uint64_t i = tid; i < ntiles; i += stride) {
            tstart[i] = kNoStart;
            tlit[i] = 0;
        }
    if (blockIdx.x == 0) {
        // Thread t numbers the chunks of units [u0, u1), a contiguous run:
        // first its total (loads in batches, all in flight together), then
        // a block scan, then the numbers (the same loads, now in cache).
        // Unit ids are below 2^31 and chunk is a power of two.
        const uint32_t units = payloads * g.count;
        const uint32_t per = (units + kThreads - 1) / kThreads;
        const uint32_t u0 = min(units, threadIdx.x * per), u1 = min(units, u0 + per);
        const uint32_t lg = 31u - (uint32_t)__clz(chunk);
        constexpr uint32_t kBatch = 8;
        auto chunks_of = [&](uint32_t a, uint64_t (&L)[kBatch], uint64_t (&B)[kBatch]) {
#pragma unroll
            for (uint32_t k = 0; k < kBatch; ++k) {
                L[k] = 0;
                B[k] = 0;
                if (a + k < u1) {
                    B[k] = quartic_len(load_seg(g, (a + k) % g.count).n);
                    L[k] = in_lens[a + k];
                }
            }
#pragma unroll
            for (uint32_t k = 0; k < kBatch; ++k) L[k] = min(L[k], B[k]);
        };
        uint32_t mine = 0;
        uint64_t sum_l = 0, sum_b = 0;
        for (uint32_t a = u0; a < u1; a += kBatch) {
            uint64_t L[kBatch], B[kBatch];
            chunks_of(a, L, B);
#pragma unroll
            for (uint32_t k = 0; k < kBatch; ++k)
                if (a + k < u1) {
                    mine += max(1u, (uint32_t)((L[k] + chunk - 1) >> lg));
                    sum_l += L[k];
                    sum_b += B[k];
                }
        }
        uint32_t carry;
        uint32_t first = block_excl_sum(mine, s_u, &carry);
        for (uint32_t a = u0; a < u1; a += kBatch) {
            uint64_t L[kBatch], B[kBatch];
            chunks_of(a, L, B);
#pragma unroll
            for (uint32_t k = 0; k < kBatch; ++k)
                if (a + k < u1) {
                    const uint32_t u = a + k;
                    const uint32_t rc = max(1u, (uint32_t)((L[k] + chunk - 1) >> lg));
                    dec_first[u] = first;
                    tickets[u] = 0;
                    fill_words(dec_map + first, rc, u | (rc > 1 ? kMulti : 0u));
                    first += rc;
                }
        }
        if (hint) {
            for (int d = 32; d >= 1; d >>= 1) {
                sum_l += __shfl_xor(sum_l, d, 64);
                sum_b += __shfl_xor(sum_b, d, 64);
            }
            if (lane_id() == 0) {
                s_d[0][wave_id()] = sum_l;
                s_d[1][wave_id()] = sum_b;
            }
            __syncthreads();
            if (threadIdx.x == 0) {
                uint64_t tl = 0, tb = 0;
                for (int w = 0; w < kWaves; ++w) {
                    tl += s_d[0][w];
                    tb += s_d[1][w];
                }
                *hint = kDenseDen * tl > dense_num * tb ? 1u : 0u;
            }
        }
        if (threadIdx.x == 0) {
            ctrl[3] = carry;  // decoder chunks
            *status = TLC_OK;
        }
    }
}

// What k_decode does with a chunk once it knows where the chunk's bytes land.
enum DecodeMode {
    kDecodeWrite = 0,    // sparse decompress: nonzero codes written over k_prep's zero fill
    kDecodeAdd = 1,      // accumulate one payload: nonzero codes added to acc in place
    kDecodeRecord = 2,   // dense decompress and accumulate-many: tile starts and literal flags
};

// Sum of the expansion lengths of the four bytes of w (1 for a literal, b -
// 241 for a run code b >= 243): with S = sum of the bytes and D = sum of
// |b - 242| (two v_sad_u8), S + D - 4*242 = 2 * sum of (b - 242) over the
// run codes.
__device__ __forceinline__ uint32_t runs_len4(uint32_t w) {
    const uint32_t sum = __builtin_amdgcn_sad_u8(w, 0u, 0u), dev = __builtin_amdgcn_sad_u8(w, 0xF2F2F2F2u, 0u);
    return 4u + ((sum + dev - 4u * 242u) >> 1);
}

// Bit 8i+7 set when byte i of w is a literal holding a nonzero code (not a
// run code >= 243, not 121): a byte is >= 243 when its top bit is set and
// its low seven bits plus 13 carry into bit 7; it is 121 when it xor 0x79 is
// zero (bit 7 of ~(((t & 0x7F) + 0x7F) | t | 0x7F)).  No carry crosses a byte.
__device__ __forceinline__ uint32_t literal_bits(uint32_t w) {
    const uint32_t run = ((w & 0x7F7F7F7Fu) + 0x0D0D0D0Du) & w & 0x80808080u;
    const uint32_t t = w ^ 0x79797979u;
    const uint32_t zero = ~(((t & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | t | 0x7F7F7F7Fu);
    return ~(run | zero) & 0x80808080u;
}

// One block per stream chunk (BPL bytes per lane: 4 KiB, or 16 KiB for the
// record pass over many payloads, where fewer, larger chunks take fewer
// rounds of the resident grid): expansion lengths,
// block scan, look-back across the unit's chunks for the quartic byte index
// of the chunk, then the work of Mode (one instantiation each, so that each
// keeps only its own registers).  Record mode writes payload p's tile
// records at p * rstride.  Only the chunks of units [u_lo, u_hi) are taken
// (u_hi == kToEnd: through the last unit), so that the payloads of one set-up
// can be decoded one launch after the other.
template <int Mode, uint32_t BPL>
__global__ __launch_bounds__(kThreads) void k_decode(GroupView g, const uint8_t* __restrict__ in,
                                                     uint64_t in_stride, uint64_t rstride,
                                                     const uint64_t* __restrict__ in_lens,
                                                     const float* __restrict__ scales, float s,
                                                     float* __restrict__ y, uint64_t* __restrict__ tstart,
                                                     uint32_t* __restrict__ tlit, uint64_t* __restrict__ flags,
                                                     const uint32_t* __restrict__ dec_map,
                                                     const uint32_t* __restrict__ dec_first,
                                                     uint32_t* __restrict__ tickets, const uint32_t* __restrict__ ctrl,
                                                     int* __restrict__ status, uint32_t u_lo, uint32_t u_hi) {
    __shared__ uint32_t s_u[kWaves];
    __shared__ uint32_t s_chunk, s_ok;
    __shared__ uint64_t s_base;
    // The real chunk count is only known on the device: the grid is capped
    // near what the GPU holds at once and blocks loop over the chunks.
    // Chunks are numbered in unit order, so a unit range is a chunk range.
    const uint32_t lo = u_lo ? dec_first[u_lo] : 0u;
    const uint32_t hi = u_hi == kToEnd ? ctrl[3] : dec_first[u_hi];
    for (uint32_t slot = lo + blockIdx.x; slot < hi; slot += gridDim.x) {
        if (slot != lo + blockIdx.x) __syncthreads();  // s_chunk / s_base of the previous chunk are read
        // A unit with several chunks hands them out in ticket order from its
        // own counter, so that the look-back only ever waits for blocks that
        // already hold a smaller ticket (and are working on that chunk).
        const uint32_t ent = dec_map[slot];
        const uint32_t u = ent & ~kMulti;
        const uint32_t t = u % g.count, p = u / g.count;
        if (threadIdx.x == 0) s_chunk = (ent & kMulti) ? atomicAdd(tickets + u, 1u) : 0u;  // in flight with the loads
        const uint32_t c0 = dec_first[u];
        const float msc = scales[u];
        const Seg sg = load_seg(g, t);
        const uint32_t n = sg.n;
        const uint64_t B = quartic_len(n);
        const uint64_t L_in = in_lens[u];
        const uint64_t L = min(L_in, B);
        const uint8_t* const sp = in + (uint64_t)p * in_stride;  // payload p's stream buffer
        __syncthreads();
        const uint32_t lc = s_chunk;
        const uint32_t c = c0 + lc;
        if (L_in > B && lc == 0 && threadIdx.x == 0) raise_status(status, TLC_ERR_CORRUPT);
        constexpr uint32_t kChunkT = kThreads * BPL;
        const uint64_t start = (uint64_t)lc * kChunkT;
        if (start >= L) {
            // only an empty stream gets here (chunk 0 of a unit with L == 0),
            // which is corrupt because ceil(n/5) >= 1
            if (threadIdx.x == 0) raise_status(status, TLC_ERR_CORRUPT);
            continue;
        }
        const uint32_t cnt = (uint32_t)min((uint64_t)kChunkT, L - start);
        const uint8_t* const pb = sp + sg.stream_off + start;
        const uint32_t off = BPL * threadIdx.x;
        const uint32_t nv = cnt > off ? min(BPL, cnt - off) : 0u;
        uint32_t wd[BPL / 4];
#pragma unroll
        for (uint32_t i = 0; i < BPL / 4; ++i) wd[i] = 0u;
        if (nv == BPL && ((reinterpret_cast<uintptr_t>(pb + off) & 15) == 0)) {
#pragma unroll
            for (uint32_t q = 0; q < BPL / 16; ++q) {
                const uint4 v = reinterpret_cast<const uint4*>(pb + off)[q];
                wd[4 * q] = v.x;
                wd[4 * q + 1] = v.y;
                wd[4 * q + 2] = v.z;
                wd[4 * q + 3] = v.w;
            }
        } else {
            for (uint32_t i = 0; i < nv; ++i) wd[i >> 2] |= (uint32_t)pb[off + i] << (8 * (i & 3));
        }
        uint32_t tsum = 0, nlit = 0;
        if (nv == BPL) {  // whole words: four bytes at a time
#pragma unroll
            for (uint32_t k = 0; k < BPL / 4; ++k) {
                tsum += runs_len4(wd[k]);
                if (Mode != kDecodeRecord) nlit += __popc(literal_bits(wd[k]));
            }
        } else {
            for (uint32_t i = 0; i < nv; ++i) {
                const uint32_t byte = (wd[i >> 2] >> (8 * (i & 3))) & 255u;
                tsum += byte < 243u ? 1u : byte - kRunBase;
                nlit += (byte < 243u && byte != kZero) ? 1u : 0u;
            }
        }
        uint32_t csum;
        const uint32_t texcl = block_excl_sum(tsum, s_u, &csum);

        if (threadIdx.x < 64) {
            uint64_t base = 0;
            uint32_t ok = 1;
            if (lc == 0) {
                if (threadIdx.x == 0) publish(flags, c, kPrefix, csum);
            } else {
                if (threadIdx.x == 0) publish(flags, c, kAggregate, csum);
                ok = look_back(flags, c, c0, 0, SumCompose(), &base) ? 1u : 0u;
                if (threadIdx.x == 0) publish(flags, c, ok ? kPrefix : kPoison, base + csum);
            }
            if (threadIdx.x == 0) {
                s_base = base;
                s_ok = ok;
            }
        }
        __syncthreads();
        const uint64_t base = s_base;
        if (!s_ok) {
            if (threadIdx.x == 0) raise_status(status, TLC_ERR_INTERNAL);
            continue;
        }
        if (threadIdx.x == 0 && start + cnt == L && base + csum != B) raise_status(status, TLC_ERR_CORRUPT);
        uint64_t pos = base + texcl;
        bool bad = false;
        if (Mode == kDecodeWrite || Mode == kDecodeAdd) {
            if (nlit) {  // lanes whose bytes hold no nonzero code write nothing
                float* const yy = y + sg.elem_off;
                const float ms = msc * s;
#pragma unroll
                for (uint32_t i = 0; i < BPL; ++i) {
                    const uint32_t byte = (wd[i >> 2] >> (8 * (i & 3))) & 255u;
                    if (i < nv) {
                        if (byte < 243u) {
                            if (pos >= B) {
                                bad = true;
                            } else if (byte != kZero) {
                                uint32_t rest = byte;
#pragma unroll
                                for (uint32_t d = 0; d < 5; ++d) {
                                    const uint32_t digit = rest % 3u;
                                    rest /= 3u;
                                    const uint64_t e = 5u * pos + d;
                                    if (digit != 1u && e < n) {
                                        const float val = (float)((int)digit - 1) * ms;
                                        yy[e] = Mode == kDecodeAdd ? yy[e] + val : val;
                                    }
                                }
                            }
                            pos += 1;
                        } else {
                            pos += byte - kRunBase;
                        }
                    }
                }
            }
        } else {
            // A lane's BPL bytes expand to at most 14 BPL < 1024 quartic
            // bytes, so at most one tile boundary (a multiple of 1024) falls
            // inside them, d quartic bytes after the lane's first; the lane's
            // literal bytes lie in the tiles before and after it.
            static_assert(BPL * (255u - kRunBase) < kETileBytes, "one tile boundary per lane");
            const uint64_t p0 = base + texcl;
            const uint32_t d = (uint32_t)((kETileBytes - p0 % kETileBytes) % kETileBytes);
            const uint32_t lim = (uint32_t)min<uint64_t>(B - min(B, p0), 1u << 16);  // quartic bytes left in the tensor
            uint32_t bi = BPL, bskip = 0;  // the byte whose expansion holds the boundary
            bool lit_lo = false, lit_hi = false;
            if (nv == BPL) {
                // the word holding the boundary, from the words' length sums;
                // literals per word; then the byte within that word.  A
                // literal past the tensor's end makes the stream longer than
                // its quartic length, which the chunk that ends it reports.
                uint32_t rel = 0, relc = 0, wc = 0, kc = BPL / 4;
                uint32_t before = 0, after = 0;  // literal bits of the words before and after word kc
#pragma unroll
                for (uint32_t k = 0; k < BPL / 4; ++k) {
                    const uint32_t len = runs_len4(wd[k]);
                    const uint32_t lb = literal_bits(wd[k]);
                    const bool here = kc == BPL / 4 && d < rel + len;
                    if (here) {
                        kc = k;
                        relc = rel;
                        wc = wd[k];
                    }
                    if (kc == BPL / 4) before |= lb;
                    else if (!here) after |= lb;
                    rel += len;
                }
                if (kc < BPL / 4) {
                    uint32_t r = relc, j = 4;
#pragma unroll
                    for (uint32_t q = 0; q < 4; ++q) {
                        const uint32_t byte = (wc >> (8 * q)) & 255u;
                        const uint32_t len = byte < 243u ? 1u : byte - kRunBase;
                        if (j == 4 && d < r + len) {
                            j = q;
                            bskip = d - r;
                        }
                        r += len;
                    }
                    bi = 4 * kc + j;
                    const uint32_t lc = literal_bits(wc);
                    const uint32_t lo_mask = j == 0 ? 0u : (0xFFFFFFFFu >> (32 - 8 * j));
                    lit_lo = (before | (lc & lo_mask)) != 0u;
                    lit_hi = (after | (lc & ~lo_mask)) != 0u;
                } else {
                    lit_lo = before != 0u;
                }
            } else {
                uint32_t rel = 0;
                for (uint32_t i = 0; i < nv; ++i) {
                    const uint32_t byte = (wd[i >> 2] >> (8 * (i & 3))) & 255u;
                    const uint32_t len = byte < 243u ? 1u : byte - kRunBase;
                    if (d >= rel && d < rel + len) {
                        bi = i;
                        bskip = d - rel;
                    }
                    if (byte < 243u && byte != kZero) {
                        lit_lo |= rel < d;
                        lit_hi |= rel >= d;
                    }
                    rel += len;
                }
            }
            uint64_t* const ts = tstart + (uint64_t)p * rstride + sg.etile0;
            uint32_t* const tl = tlit + (uint64_t)p * rstride + sg.etile0;
            if (bi < BPL && d < lim) ts[(p0 + d) / kETileBytes] = tile_start(start + off + bi, bskip);
            // flags only for tiles of this tensor
            if (lit_lo && lim > 0) tl[p0 / kETileBytes] = 1u;
            if (lit_hi && d < lim) tl[(p0 + d) / kETileBytes] = 1u;
        }
        if (bad) raise_status(status, TLC_ERR_CORRUPT);
    }
}

// Unit handled by block b of a grid of 8 * ceil(units / 8) blocks (a result
// >= units means none).  Blocks are dispatched round-robin over the 8 XCDs,
// so this gives each XCD a contiguous eighth of the units: large per-block
// stores then reach ~6.2 TB/s on MI355X, against ~5.5 TB/s in plain order.
__device__ __forceinline__ uint32_t xcd_unit(uint32_t b, uint32_t units) {
    const uint32_t q = (units + 7) / 8;
    return (b % 8) * q + b / 8;
}
uint32_t xcd_grid(uint64_t units) { return (uint32_t)((units + 7) / 8 * 8); }

// One wavefront per encode tile (5120 elements, 1024 quartic bytes), four per
// block, with no block barrier: every element of the tile is written once,
// y = q * (M*s), with streaming 16-byte stores (as the zero fill), so
// decompress writes each line of y once (a zero fill with the nonzero values
// scattered over it afterwards wrote every line that holds a nonzero code
// twice).  A tile k_decode found no nonzero code in is written without
// reading the stream.  Otherwise its stream bytes, from the start k_decode
// recorded, are staged in LDS with aligned 16-byte loads, re-read 16 per lane
// in stream order, and expanded into the tile's codes (one int8 per element,
// same LDS slice).
__global__ __launch_bounds__(kThreads) void k_expand(GroupView g, uint32_t etiles, const uint8_t* __restrict__ in,
                                                     const uint64_t* __restrict__ in_lens,
                                                     const float* __restrict__ scales, float s,
                                                     const uint64_t* __restrict__ tstart,
                                                     const uint32_t* __restrict__ tlit, float* __restrict__ y,
                                                     int* __restrict__ status) {
    __shared__ __align__(16) int8_t s_codes[kWaves * kETile];
    const int lane = lane_id();
    const uint32_t wave = __builtin_amdgcn_readfirstlane(wave_id());
    const uint32_t e = xcd_unit(blockIdx.x, (etiles + kWaves - 1) / kWaves) * kWaves + wave;
    if (e >= etiles) return;
    int8_t* const sq = s_codes + wave * kETile;
    const uint32_t gi = etile_owner(g, e);
    const uint64_t ts = tstart[e];
    const uint64_t tn = e + 1 < etiles ? tstart[e + 1] : kNoStart;
    const bool has_lit = tlit[e] != 0u;
    const Seg sg = load_seg(g, gi);
    const float ms = scales[gi] * s;
    const uint64_t L_in = in_lens[gi];
    if (ts == kNoStart) {  // the stream never reached this tile
        if (lane == 0) raise_status(status, TLC_ERR_CORRUPT);
        return;
    }
    const uint32_t j = e - sg.etile0;
    const uint32_t nel = min(kETile, sg.n - j * kETile);
    if (has_lit) {
        const uint64_t B = quartic_len(sg.n);
        const uint32_t need = (uint32_t)min((uint64_t)kETileBytes, B - (uint64_t)j * kETileBytes);
        const uint64_t sb = ts & 0xFFFFFFFFull, skip = ts >> 32;
        // bytes sb .. eb-1: at most 1024 (each covers at least one quartic
        // byte), none past the byte where the tensor's next tile begins
        uint64_t eb = min(min(L_in, B), sb + kETileBytes);
        if ((uint64_t)(j + 1) * kETileBytes < B && tn != kNoStart) eb = min(eb, (tn & 0xFFFFFFFFull) + 1);
        // 16-byte chunks c = 0..64 from the one holding byte sb; each one
        // loaded holds a byte of the tile, so it lies in a readable page
        const uint8_t* const p = in + sg.stream_off + sb;
        const uint8_t* const pend = in + sg.stream_off + eb;
        const uint4* const a16 = reinterpret_cast<const uint4*>(reinterpret_cast<uintptr_t>(p) & ~(uintptr_t)15);
        const uint32_t o = (uint32_t)(p - reinterpret_cast<const uint8_t*>(a16));  // 0..15, wave-uniform
        uint4 c0 = make_uint4(0u, 0u, 0u, 0u), c1 = c0;
        if (reinterpret_cast<const uint8_t*>(a16 + lane) < pend) c0 = a16[lane];
        if (lane == 0 && reinterpret_cast<const uint8_t*>(a16 + 64) < pend) c1 = a16[64];
        uint4* const st16 = reinterpret_cast<uint4*>(sq);
        st16[lane] = c0;
        if (lane == 0) st16[64] = c1;
        wave_sync();
        // this lane's bytes sb + 16 lane .. + 15, from dwords 4 lane + o/4 ..
        const uint32_t* const st32 = reinterpret_cast<const uint32_t*>(sq) + 4 * lane + (o >> 2);
        uint32_t w5[5];
#pragma unroll
        for (int i = 0; i < 5; ++i) w5[i] = st32[i];
        uint32_t wd[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) wd[i] = __builtin_amdgcn_alignbyte(w5[i + 1], w5[i], o & 3u);
        const uint64_t have = eb - sb;
        const uint32_t nv = (uint32_t)min<uint64_t>(16u, have > 16u * lane ? have - 16u * lane : 0u);
        uint32_t tsum = 0;
#pragma unroll
        for (uint32_t i = 0; i < 16; ++i) {
            const uint32_t byte = (wd[i >> 2] >> (8 * (i & 3))) & 255u;
            uint32_t len = i < nv ? (byte < 243u ? 1u : byte - kRunBase) : 0u;
            if (lane == 0 && i == 0) len = len > skip ? len - (uint32_t)skip : 0u;
            tsum += len;
        }
        uint32_t tot;
        uint32_t pos = wave_excl_sum(tsum, &tot);  // tile quartic byte of this lane's first byte
        if (tot < need && lane == 0) raise_status(status, TLC_ERR_CORRUPT);
        wave_sync();  // every lane has read the staged bytes
        uint4* const q16 = reinterpret_cast<uint4*>(sq);
#pragma unroll
        for (uint32_t k = 0; k < kETile / 16 / 64; ++k) q16[lane + 64 * k] = make_uint4(0u, 0u, 0u, 0u);
        wave_sync();
#pragma unroll
        for (uint32_t i = 0; i < 16; ++i) {
            const uint32_t byte = (wd[i >> 2] >> (8 * (i & 3))) & 255u;
            uint32_t len = i < nv ? (byte < 243u ? 1u : byte - kRunBase) : 0u;
            if (lane == 0 && i == 0) len = len > skip ? len - (uint32_t)skip : 0u;
            if (len && byte < 243u && byte != kZero && pos < need) {
                uint32_t rest = byte;
#pragma unroll
                for (uint32_t d = 0; d < 5; ++d) {
                    sq[5 * pos + d] = (int8_t)((int)(rest % 3u) - 1);
                    rest /= 3u;
                }
            }
            pos += len;
        }
        wave_sync();
    }
    // float4 group h holds tile elements 4h - mis .. 4h - mis + 3, aligned in y
    const uint64_t a = sg.elem_off + (uint64_t)j * kETile;
    const int32_t mis = (int32_t)(a & 3);
    float* const yt = y + a;
    const int32_t ng = (mis + (int32_t)nel + 3) / 4;
    for (int32_t h = lane; h < ng; h += 64) {
        const int32_t u0 = 4 * h - mis;
        int q[4] = {0, 0, 0, 0};
        if (has_lit) {
            if (mis == 0) {
                const uint32_t w = reinterpret_cast<const uint32_t*>(sq)[h];
#pragma unroll
                for (int i = 0; i < 4; ++i) q[i] = (int)(int8_t)(w >> (8 * i));
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) q[i] = u0 + i >= 0 && u0 + i < (int32_t)nel ? sq[u0 + i] : 0;
            }
        }
        const float4 v = make_float4((float)q[0] * ms, (float)q[1] * ms, (float)q[2] * ms, (float)q[3] * ms);
        if (u0 >= 0 && u0 + 4 <= (int32_t)nel) {
            store_stream(reinterpret_cast<f4*>(yt + u0), f4{v.x, v.y, v.z, v.w});
        } else {
            if (u0 >= 0 && u0 < (int32_t)nel) yt[u0] = v.x;
            if (u0 + 1 >= 0 && u0 + 1 < (int32_t)nel) yt[u0 + 1] = v.y;
            if (u0 + 2 >= 0 && u0 + 2 < (int32_t)nel) yt[u0 + 2] = v.z;
            if (u0 + 3 < (int32_t)nel) yt[u0 + 3] = v.w;
        }
    }
}

// Payload l's 64-bit value held by lane l, in scalar registers (l uniform).
__device__ __forceinline__ uint64_t readlane64(uint64_t v, uint32_t l) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, (int)l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), (int)l);
    return (uint64_t)hi << 32 | lo;
}

// Inclusive prefix sum over the wavefront with DPP moves: shifts of 1, 2, 4
// and 8 lanes within each row of 16, then the last lane of row 0 added to
// row 1 and that of row 2 to row 3 (row_bcast:15), then the last lane of
// row 1 added to rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ uint32_t wave_incl_sum_dpp(uint32_t x) {
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, true);  // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, true);  // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, true);  // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, true);  // row_shr:8
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15, rows 1 and 3
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31, rows 2 and 3
    return x;
}

// The five codes of a quartic byte as 2-bit fields, first element lowest:
// bit 2d is set when code d is nonzero, bit 2d+1 when the value it adds is
// negative: q = -1 adds -M*s, and q = 0 adds -0.0, which leaves every
// finite value's bits unchanged (x + -0.0 = x, -0.0 included).
__device__ __forceinline__ uint32_t quartic_fields(uint32_t byte) {
    uint32_t pat = 0;
    for (uint32_t d = 0; d < 5; ++d) {
        const uint32_t digit = byte % 3u;
        byte /= 3u;
        pat |= (digit == 1u ? 2u : digit == 2u ? 1u : 3u) << (2 * d);
    }
    return pat;
}

// Where an encode tile's bytes lie in a payload's stream, from the tile's
// start record: from byte sb (whose expansion holds `skip` quartic bytes of
// the tile before) to the byte where the tensor's next tile begins (a run
// can straddle), at most 1024 bytes (each covers at least one quartic
// byte), cut at the stream's end.
struct TileBytes {
    uint64_t sb, have;
    uint32_t skip;
};
__device__ __forceinline__ TileBytes tile_bytes(uint64_t ts, uint64_t tn, uint64_t L, uint64_t B, bool last_tile) {
    TileBytes t;
    t.sb = ts & 0xFFFFFFFFull;
    uint64_t eb = min(min(L, B), t.sb + kETileBytes);
    if (!last_tile && tn != kNoStart) eb = min(eb, (tn & 0xFFFFFFFFull) + 1);
    t.have = eb > t.sb ? eb - t.sb : 0;
    t.skip = (uint32_t)(ts >> 32);
    return t;
}

// Dword w of the 4-byte-aligned window holding a tile's bytes (lane l of
// block b loads dword 64 b + l), or 0 past the bytes; a dword loaded holds
// a byte of the tile, so it lies in a readable page.
__device__ __forceinline__ uint32_t tile_dword(const uint8_t* tensor_stream, const TileBytes& t, uint32_t w) {
    const uint8_t* const a4 = tensor_stream + (t.sb & ~3ull);
    const uint64_t o4 = t.sb & 3u;
    return 4ull * w < o4 + t.have ? reinterpret_cast<const uint32_t*>(a4)[w] : 0u;
}

// Where encode tile e lies (wave-uniform).
struct ApplyTile {
    uint64_t a0;    // group element of its first value
    uint64_t soff;  // stream slot of its tensor
    uint64_t B;     // quartic bytes of its tensor
    uint32_t gi, nel, need;
    int32_t mis;    // a0 mod 4
    uint32_t last;  // 1 for the tensor's last tile
};
__device__ __forceinline__ ApplyTile apply_tile(const Seg& sg, uint32_t gi, uint32_t e) {
    ApplyTile t;
    t.gi = gi;
    const uint32_t j = e - sg.etile0;
    t.nel = min(kETile, sg.n - j * kETile);
    t.B = quartic_len(sg.n);
    t.need = (uint32_t)min((uint64_t)kETileBytes, t.B - (uint64_t)j * kETileBytes);
    t.last = (uint64_t)(j + 1) * kETileBytes >= t.B ? 1u : 0u;
    t.a0 = sg.elem_off + (uint64_t)j * kETile;
    t.mis = (int32_t)(t.a0 & 3);
    t.soff = sg.stream_off;
    return t;
}

// Payload `lane`'s record of tile e (lanes past the payloads hold none).
struct ApplyRec {
    uint64_t ts, tn, L;
    uint32_t lit;
    float ms;
};
__device__ __forceinline__ ApplyRec apply_rec(const GroupView& g, uint32_t etiles, uint32_t payloads, uint32_t e,
                                              uint32_t gi, const uint64_t* tstart, const uint32_t* tlit,
                                              const uint64_t* in_lens, const float* scales, float s) {
    ApplyRec r;
    r.ts = kNoStart;
    r.tn = kNoStart;
    r.L = 0;
    r.lit = 0;
    r.ms = 0.0f;
    const uint32_t lane = (uint32_t)lane_id();
    if (lane < payloads) {
        const uint64_t i = (uint64_t)lane * etiles + e;
        const uint64_t u = (uint64_t)lane * g.count + gi;
        r.ts = tstart[i];
        if (e + 1 < etiles) r.tn = tstart[i + 1];
        r.lit = tlit[i];
        r.L = in_lens[u];
        r.ms = scales[u] * s;
    }
    return r;
}

// acc += q_p * (M_p*s) for payloads p = 0 .. payloads-1 in that order, only
// where q_p != 0 (an element no payload touches keeps its bits, -0.0
// included).  Persistent wavefronts (one per block), each over a contiguous
// range of encode tiles (up to 5120 elements of one tensor), the ranges
// contiguous per XCD.  For each tile, lane p reads payload p's record:
// where the tile begins in its stream, and whether the bytes there hold a
// nonzero code; a tile where no payload has one is not touched.  Otherwise
// the tile of acc is copied into LDS (tile element u at word u + mis, so
// that float4 group h is LDS words 4h .. 4h+3).  Then, one payload after the
// other, its bytes for the tile are walked 64 at a time, one per lane
// (ds_bpermute from the lanes that loaded them as dwords, 256 bytes per
// load): a wave scan of their expansion lengths gives each byte's quartic
// position, and each nonzero code of a literal byte is added to its element
// with an LDS float atomic add: it returns nothing, so nothing waits for it,
// and a wave's LDS operations execute in order, so the payloads' adds to an
// element follow the payload order (the add rounds exactly as v_add_f32,
// denormals included, measured on MI355X over 16M operand pairs).
// Neighbouring lanes hold neighbouring bytes, so their elements fall in
// different LDS banks.  The tile is written back once.  While one tile is
// decoded, the next tile's acc and its payloads' first 256 bytes (8
// payloads' worth) are in flight, and the records of the one after.
constexpr uint32_t kApplyFetch = 8;                           // payloads whose first bytes are fetched ahead
constexpr uint32_t kApplyVec = ((kETile + 6) / 4 + 63) / 64;  // float4 groups per lane: 21
constexpr uint32_t kApplyWords = (kETile + 3 + 3) / 4 * 4;    // LDS words of a tile: 5124

__device__ __forceinline__ void apply_fetch(const ApplyTile& t, const ApplyRec& r, uint64_t lits, const float* acc,
                                            const uint8_t* in, uint64_t in_stride, f4 (&v)[kApplyVec],
                                            uint32_t (&dw)[kApplyFetch]) {
    const int lane = lane_id();
    const float* const at = acc + t.a0;
    const int32_t ng = (t.mis + (int32_t)t.nel + 3) / 4;
    if (lits && t.mis == 0 && t.nel == kETile) {  // a whole aligned tile: 20 float4 per lane
#pragma unroll
        for (uint32_t k = 0; k < kApplyVec; ++k)
            v[k] = k < kETile / 256 ? __builtin_nontemporal_load(reinterpret_cast<const f4*>(at) + lane + 64 * k)
                                    : f4{0.0f, 0.0f, 0.0f, 0.0f};
    } else {
#pragma unroll
        for (uint32_t k = 0; k < kApplyVec; ++k) {
            const int32_t h = lane + 64 * (int32_t)k;
            const int32_t u0 = 4 * h - t.mis;
            v[k] = f4{0.0f, 0.0f, 0.0f, 0.0f};
            if (lits && h < ng) {
                if (u0 >= 0 && u0 + 4 <= (int32_t)t.nel) {
                    v[k] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(at + u0));
                } else {
#pragma unroll
                    for (int32_t i = 0; i < 4; ++i)
                        if (u0 + i >= 0 && u0 + i < (int32_t)t.nel) v[k][i] = at[u0 + i];
                }
            }
        }
    }
#pragma unroll
    for (uint32_t k = 0; k < kApplyFetch; ++k) {
        dw[k] = 0u;
        if (lits & (1ull << k)) {
            const TileBytes tb =
                tile_bytes(readlane64(r.ts, k), readlane64(r.tn, k), readlane64(r.L, k), t.B, t.last != 0u);
            dw[k] = tile_dword(in + (uint64_t)k * in_stride + t.soff, tb, (uint32_t)lane);
        }
    }
}

__global__ __launch_bounds__(64, 2) void k_apply(GroupView g, uint32_t etiles, uint32_t nwaves, uint32_t payloads,
                                                 const uint8_t* __restrict__ in, uint64_t in_stride,
                                                 const uint64_t* __restrict__ in_lens,
                                                 const float* __restrict__ scales, float s,
                                                 const uint64_t* __restrict__ tstart,
                                                 const uint32_t* __restrict__ tlit, float* __restrict__ acc,
                                                 int* __restrict__ status) {
    __shared__ __align__(16) float s_acc[kApplyWords];
    __shared__ uint16_t s_tab[256];
    const int lane = lane_id();
    const uint32_t w = xcd_unit(blockIdx.x, nwaves);
    if (w >= nwaves) return;
    const uint32_t per = (etiles + nwaves - 1) / nwaves;
    const uint32_t e_end = min(etiles, (w + 1) * per);
    uint32_t e = w * per;
    if (e >= e_end) return;
    for (uint32_t t = (uint32_t)lane; t < 243u; t += 64u) s_tab[t] = (uint16_t)quartic_fields(t);

    // the tensor of the furthest tile looked up so far; tiles are in tensor
    // order, so the next one is the same tensor or the one after
    uint32_t gi_f = etile_owner(g, e);
    Seg sg_f = load_seg(g, gi_f);
    auto tile_at = [&](uint32_t te) {
        while (gi_f + 1 < g.count && te - sg_f.etile0 >= etiles_of(sg_f.n)) sg_f = load_seg(g, ++gi_f);
        return apply_tile(sg_f, gi_f, te);
    };
    ApplyTile t0 = tile_at(e);
    ApplyRec r0 = apply_rec(g, etiles, payloads, e, t0.gi, tstart, tlit, in_lens, scales, s);
    uint64_t lits0 = __ballot(r0.lit != 0u && r0.ts != kNoStart);
    f4 v[kApplyVec];  // the acc of the tile about to be decoded, on its way to LDS
    uint32_t d0[kApplyFetch];
    apply_fetch(t0, r0, lits0, acc, in, in_stride, v, d0);
    bool has1 = e + 1 < e_end;
    ApplyTile t1 = t0;
    ApplyRec r1 = r0;
    if (has1) {
        t1 = tile_at(e + 1);
        r1 = apply_rec(g, etiles, payloads, e + 1, t1.gi, tstart, tlit, in_lens, scales, s);
    }
    // ds_bpermute byte addresses: byte 64 q + l of a 256-byte window is byte
    // l & 3 of the dword of lane 16 q + l / 4
    const uint32_t src_lane = (uint32_t)lane >> 2, src_shift = 8u * ((uint32_t)lane & 3u);
    for (;;) {
        if (__ballot((uint32_t)lane < payloads && r0.ts == kNoStart) && lane == 0)
            raise_status(status, TLC_ERR_CORRUPT);  // a stream that never reached this tile
        const int32_t ng = (t0.mis + (int32_t)t0.nel + 3) / 4;
        const bool whole = t0.mis == 0 && t0.nel == kETile;  // 20 float4 per lane, no partial group
        if (lits0) {
#pragma unroll
            for (uint32_t k = 0; k < kApplyVec; ++k) {
                const int32_t h = lane + 64 * (int32_t)k;
                if (whole ? k < kETile / 256 : h < ng) reinterpret_cast<f4*>(s_acc)[h] = v[k];
            }
        }
        wave_sync();
        // the next tile's data and the records of the one after, in flight
        // while this tile is decoded
        uint64_t lits1 = 0;
        uint32_t d1[kApplyFetch];
        if (has1) {
            lits1 = __ballot(r1.lit != 0u && r1.ts != kNoStart);
            apply_fetch(t1, r1, lits1, acc, in, in_stride, v, d1);
        }
        const bool has2 = e + 2 < e_end;
        ApplyTile t2 = t1;
        ApplyRec r2 = r1;
        if (has2) {
            t2 = tile_at(e + 2);
            r2 = apply_rec(g, etiles, payloads, e + 2, t2.gi, tstart, tlit, in_lens, scales, s);
        }
        if (lits0) {
            for (uint32_t p = 0; p < payloads; ++p) {
                if (!((lits0 >> p) & 1u)) continue;
                const uint32_t mb = (uint32_t)__builtin_amdgcn_readlane(__builtin_bit_cast(int, r0.ms), (int)p);
                const uint8_t* const ps = in + (uint64_t)p * in_stride + t0.soff;
                const TileBytes tb = tile_bytes(readlane64(r0.ts, p), readlane64(r0.tn, p), readlane64(r0.L, p), t0.B,
                                                t0.last != 0u);
                const uint32_t o4 = (uint32_t)(tb.sb & 3u);
                const uint32_t span = o4 + (uint32_t)tb.have;  // window bytes to walk
                uint32_t carry = 0;                             // quartic bytes of the tile so far
                uint32_t cur = 0;
#pragma unroll
                for (uint32_t k = 0; k < kApplyFetch; ++k)
                    if (p == k) cur = d0[k];
                // rounds of 64 window bytes, one per lane, as many as the bytes need
                for (uint32_t r = 0; 64u * r < span; ++r) {
                    if ((r & 3u) == 0 && (r > 0 || p >= kApplyFetch)) cur = tile_dword(ps, tb, 16u * r + (uint32_t)lane);
                    const uint32_t wpos = 64u * r + (uint32_t)lane;  // window byte of this lane
                    const uint32_t word =
                        (uint32_t)__builtin_amdgcn_ds_bpermute((int)((16u * (r & 3u) + src_lane) * 4u), (int)cur);
                    const uint32_t byte = (word >> src_shift) & 255u;
                    const uint32_t pat = s_tab[min(byte, 242u)];
                    uint32_t len = wpos >= o4 && wpos < span ? (byte < 243u ? 1u : byte - kRunBase) : 0u;
                    if (wpos == o4) len = len > tb.skip ? len - tb.skip : 0u;
                    const uint32_t incl = wave_incl_sum_dpp(len);
                    const uint32_t pos = carry + incl - len;  // tile quartic byte of this lane's byte
                    carry += (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
                    // each nonzero code of a literal byte: an LDS float add, no
                    // return (in order within the wave, rounded as v_add_f32)
                    if (len != 0u && byte < 243u && byte != kZero && pos < t0.need) {
                        float* const el = s_acc + 5u * pos + (uint32_t)t0.mis;
#pragma unroll
                        for (uint32_t d = 0; d < 5; ++d)
                            if ((pat >> (2 * d)) & 1u)
                                atomicAdd(el + d, __builtin_bit_cast(float, mb | (((pat >> (2 * d + 1)) & 1u) << 31)));
                    }
                }
                if (carry < t0.need && lane == 0) raise_status(status, TLC_ERR_CORRUPT);
            }
            wave_sync();  // every element's sum is in LDS
            float* const at = acc + t0.a0;
            if (whole) {
#pragma unroll
                for (uint32_t k = 0; k < kETile / 256; ++k)
                    __builtin_nontemporal_store(reinterpret_cast<const f4*>(s_acc)[lane + 64 * k],
                                                reinterpret_cast<f4*>(at) + lane + 64 * k);
            } else {
#pragma unroll
                for (uint32_t k = 0; k < kApplyVec; ++k) {
                    const int32_t h = lane + 64 * (int32_t)k;
                    const int32_t u0 = 4 * h - t0.mis;
                    if (h < ng) {
                        const f4 v = reinterpret_cast<const f4*>(s_acc)[h];
                        if (u0 >= 0 && u0 + 4 <= (int32_t)t0.nel) {
                            __builtin_nontemporal_store(v, reinterpret_cast<f4*>(at + u0));
                        } else {
#pragma unroll
                            for (int32_t i = 0; i < 4; ++i)
                                if (u0 + i >= 0 && u0 + i < (int32_t)t0.nel) at[u0 + i] = v[i];
                        }
                    }
                }
            }
        }
        if (!has1) break;
        ++e;
        t0 = t1;
        r0 = r1;
        lits0 = lits1;
#pragma unroll
        for (uint32_t k = 0; k < kApplyFetch; ++k) d0[k] = d1[k];
        t1 = t2;
        r1 = r2;
        has1 = has2;
    }
}

// ---------------------------------------------------------------------------
// fixed-length encodings (the ablations without zero-run encoding)

// Every encode tile's output bytes set to the encoding's byte of zero codes;
// k_quant_pack then overwrites the tiles that hold a nonzero code.  One
// wavefront per encode tile, 16 bytes per lane.
__global__ __launch_bounds__(64) void k_fixed_fill(GroupView g, uint32_t etiles, FixedOut fo) {
    const uint32_t e = blockIdx.x;
    const uint32_t gi = etile_owner(g, e);
    const Seg sg = load_seg(g, gi);
    const uint32_t TB = fixed_tile_bytes(fo.enc);
    const uint64_t j = e - sg.etile0;
    const uint32_t nb = (uint32_t)min((uint64_t)TB, fixed_len_of(sg.n, fo.enc) - j * TB);
    uint8_t* const dst = fo.out + (fo.offs ? fo.offs[gi] : 0ull) + j * TB;
    const uint8_t z = fixed_zero_byte(fo.enc);
    const uint32_t z4 = 0x01010101u * z;
    const bool al = (reinterpret_cast<uintptr_t>(dst) & 15) == 0;
    for (uint32_t c = threadIdx.x; 16 * c < nb; c += 64) {
        if (al && 16 * c + 16 <= nb) {
            *reinterpret_cast<uint4*>(dst + 16 * c) = make_uint4(z4, z4, z4, z4);
        } else {
            for (uint32_t b = 16 * c; b < min(nb, 16 * c + 16); ++b) dst[b] = z;
        }
    }
}

__global__ void k_status_ok(int* __restrict__ status) { *status = TLC_OK; }

// Decode of a fixed-length encoding: one wavefront per encode tile, four per
// block, tile ranges contiguous per XCD (as in k_expand).  Lane l reads the
// bytes of codes 80l..80l+79 (16 quartic or 20 two-bit bytes, with aligned
// vector loads when the tile's bytes start on a 16-byte boundary) and decodes
// them into LDS; y is then written with 16-byte stores, y_i = q_i * (M*s).  A
// tile whose bytes all encode zero codes skips the LDS.  A quartic byte above
// 242 or a 2-bit field of 3 sets *status = TLC_ERR_CORRUPT.
__global__ __launch_bounds__(kThreads) void k_fixed_decode(GroupView g, uint32_t etiles, int enc,
                                                           const uint8_t* __restrict__ in,
                                                           const uint64_t* __restrict__ offs,
                                                           const float* __restrict__ scales, float s,
                                                           float* __restrict__ y, int* __restrict__ status) {
    __shared__ __align__(16) int8_t s_codes[kWaves * kETile];
    const int lane = lane_id();
    const uint32_t wave = __builtin_amdgcn_readfirstlane(wave_id());
    const uint32_t e = xcd_unit(blockIdx.x, (etiles + kWaves - 1) / kWaves) * kWaves + wave;
    if (e >= etiles) return;
    int8_t* const sq = s_codes + wave * kETile;
    const uint32_t gi = etile_owner(g, e);
    const Seg sg = load_seg(g, gi);
    const uint32_t TB = fixed_tile_bytes(enc);
    const uint32_t j = e - sg.etile0;
    const uint32_t nb = (uint32_t)min((uint64_t)TB, fixed_len_of(sg.n, enc) - (uint64_t)j * TB);
    const uint32_t nel = min(kETile, sg.n - j * kETile);
    const uint8_t* const src = in + (offs ? offs[gi] : 0ull) + (uint64_t)j * TB;
    const float ms = scales[gi] * s;
    const bool two = enc == TLC_ENC_TWOBIT;
    const uint32_t nin = two ? 20u : 16u;  // bytes per lane
    const uint32_t o0 = nin * lane;
    const uint32_t zb = fixed_zero_byte(enc) * 0x01010101u;  // four zero-code bytes
    uint32_t wb[5] = {zb, zb, zb, zb, zb};
    if ((reinterpret_cast<uintptr_t>(src) & 15) == 0 && o0 + nin <= nb) {
        if (!two) {
            const uint4 v = *reinterpret_cast<const uint4*>(src + o0);
            wb[0] = v.x;
            wb[1] = v.y;
            wb[2] = v.z;
            wb[3] = v.w;
        } else {
#pragma unroll
            for (int k = 0; k < 5; ++k) wb[k] = reinterpret_cast<const uint32_t*>(src + o0)[k];
        }
    } else {
        for (uint32_t b = 0; b < nin; ++b)
            if (o0 + b < nb)
                wb[b >> 2] = (wb[b >> 2] & ~(0xFFu << (8 * (b & 3)))) | (uint32_t)src[o0 + b] << (8 * (b & 3));
    }
    bool nz = false;
#pragma unroll
    for (int k = 0; k < 5; ++k) nz |= wb[k] != zb;
    const bool any = __ballot(nz) != 0;  // wave-uniform
    if (any) {
        bool bad = false;
        uint32_t codes[20];  // 4 codes per word, as int8
#pragma unroll
        for (int i = 0; i < 20; ++i) codes[i] = 0;
        if (!two) {
#pragma unroll
            for (uint32_t b = 0; b < 16; ++b) {
                const uint32_t byte = (wb[b >> 2] >> (8 * (b & 3))) & 255u;
                bad |= byte > 242u;
                uint32_t rest = byte;
#pragma unroll
                for (uint32_t d = 0; d < 5; ++d) {
                    const uint32_t c = 5 * b + d;
                    codes[c >> 2] |= ((rest % 3u - 1u) & 0xFFu) << (8 * (c & 3));
                    rest /= 3u;
                }
            }
        } else {
#pragma unroll
            for (uint32_t b = 0; b < 20; ++b) {
                const uint32_t byte = (wb[b >> 2] >> (8 * (b & 3))) & 255u;
#pragma unroll
                for (uint32_t d = 0; d < 4; ++d) {
                    const uint32_t f = (byte >> (2 * d)) & 3u;
                    bad |= f == 3u;
                    codes[b] |= ((f - 1u) & 0xFFu) << (8 * d);
                }
            }
        }
        if (bad) raise_status(status, TLC_ERR_CORRUPT);
#pragma unroll
        for (int i = 0; i < 20; ++i) reinterpret_cast<uint32_t*>(sq)[20 * lane + i] = codes[i];
        wave_sync();
    }
    // float4 group h holds tile elements 4h - mis .. 4h - mis + 3, aligned in y
    const uint64_t a = sg.elem_off + (uint64_t)j * kETile;
    const int32_t mis = (int32_t)(a & 3);
    float* const yt = y + a;
    const int32_t ng = (mis + (int32_t)nel + 3) / 4;
    for (int32_t h = lane; h < ng; h += 64) {
        const int32_t u0 = 4 * h - mis;
        int q[4] = {0, 0, 0, 0};
        if (any) {
            if (mis == 0) {
                const uint32_t w = reinterpret_cast<const uint32_t*>(sq)[h];
#pragma unroll
                for (int i = 0; i < 4; ++i) q[i] = (int)(int8_t)(w >> (8 * i));
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) q[i] = u0 + i >= 0 && u0 + i < (int32_t)nel ? sq[u0 + i] : 0;
            }
        }
        const float4 v = make_float4((float)q[0] * ms, (float)q[1] * ms, (float)q[2] * ms, (float)q[3] * ms);
        if (u0 >= 0 && u0 + 4 <= (int32_t)nel) {
            store_stream(reinterpret_cast<f4*>(yt + u0), f4{v.x, v.y, v.z, v.w});
        } else {
            if (u0 >= 0 && u0 < (int32_t)nel) yt[u0] = v.x;
            if (u0 + 1 >= 0 && u0 + 1 < (int32_t)nel) yt[u0 + 1] = v.y;
            if (u0 + 2 >= 0 && u0 + 2 < (int32_t)nel) yt[u0 + 2] = v.z;
            if (u0 + 3 < (int32_t)nel) yt[u0 + 3] = v.w;
        }
    }
}

// ---------------------------------------------------------------------------
// bandwidth yardstick: one 16-byte load and store per lane, many small blocks,
// both streamed past the caches like the codec's own streaming accesses

// Five-plane layout helpers: tensor t (blockIdx.y) between its natural order
// (n values, plane j = elements jB .. jB + B - 1, B = ceil(n/5)) and the order
// p = 5k + j <- element k + jB (5B positions, zeros at the pads).  A block
// moves 256 byte positions k at a time through LDS: the five plane segments
// k0 + jB .. k0 + jB + 255 on one side and the 1280 consecutive positions
// 5k0 .. 5k0 + 1279 on the other, so every load and store is contiguous
// (LDS index 5(k - k0) + j: a stride of 5 words, conflict free).
template <bool kGather>
__global__ __launch_bounds__(kThreads) void k_planes(const float* __restrict__ src, const uint64_t* __restrict__ src_off,
                                                     float* __restrict__ dst, const uint64_t* __restrict__ dst_off,
                                                     const uint64_t* __restrict__ nv) {
    __shared__ float s_t[5 * kThreads];
    const uint32_t t = blockIdx.y;
    const uint64_t n = nv[t], B = (n + 4) / 5;
    const float* const s = src + src_off[t];
    float* const d = dst + dst_off[t];
    const uint32_t tid = threadIdx.x;
    for (uint64_t k0 = (uint64_t)blockIdx.x * kThreads; k0 < B; k0 += (uint64_t)gridDim.x * kThreads) {
        const uint32_t kn = (uint32_t)min<uint64_t>(kThreads, B - k0);
        if (kGather) {
#pragma unroll
            for (uint32_t j = 0; j < 5; ++j) {
                const uint64_t i = k0 + tid + j * B;
                s_t[5 * tid + j] = (tid < kn && i < n) ? s[i] : 0.0f;
            }
            __syncthreads();
#pragma unroll
            for (uint32_t r = 0; r < 5; ++r) {
                const uint32_t q = tid + kThreads * r;
                if (q < 5 * kn) d[5 * k0 + q] = s_t[q];
            }
        } else {
#pragma unroll
            for (uint32_t r = 0; r < 5; ++r) {
                const uint32_t q = tid + kThreads * r;
                if (q < 5 * kn) s_t[q] = s[5 * k0 + q];
            }
            __syncthreads();
#pragma unroll
            for (uint32_t j = 0; j < 5; ++j) {
                const uint64_t i = k0 + tid + j * B;
                if (tid < kn && i < n) d[i] = s_t[5 * tid + j];
            }
        }
        __syncthreads();  // s_t is rewritten by the next chunk
    }
}

// dst[i] = src[idx[i]]: one 4-byte read at each index (the scattered-read
// yardstick of the traffic counters).
__global__ __launch_bounds__(kThreads) void k_gather(const float* __restrict__ src, const uint32_t* __restrict__ idx,
                                                     float* __restrict__ dst, uint64_t n) {
    const uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i < n) dst[i] = src[idx[i]];
}

__global__ __launch_bounds__(kThreads) void k_copy(const float4* __restrict__ src, float4* __restrict__ dst,
                                                   uint64_t n4) {
    const uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i < n4)
        store_stream(reinterpret_cast<f4*>(dst) + i, __builtin_nontemporal_load(reinterpret_cast<const f4*>(src) + i));
}

// ---------------------------------------------------------------------------
// wire message of a group: what one worker sends in the exchange
//
// count headers of 8 bytes (header t: L_t as a little-endian uint32, then the
// bits of M_t), then the streams of tensors 0 .. count-1 back to back.  The
// 3LC page ("Proposed method") says what a compressed state change consists
// of, its scale and its byte stream; how a group's travel is this library's
// layout.  A grouped stream keeps each tensor's bytes at the start of a slot
// of ceil(n/5) bytes, so sending the message moves sum L_t + 8 count bytes
// instead of the slots' capacity.

constexpr uint32_t kWireChunk = 4096;  // stream bytes one block copies at a time (16 per lane)
constexpr uint32_t kWirePer = 16;      // tensors per thread and round of k_wire_scan

// Consecutive tensor ranges packed as messages of their own, back to back:
// range k is tensors cut[k] .. cut[k+1]-1.  With P(t) the sum of the stream
// lengths of tensors before t, message k starts at 8 cut[k] + P(cut[k]), the
// header of tensor t of range k lies at 8 t + P(cut[k]) and its stream at
// 8 cut[k+1] + P(t).  One range is the group's message.
struct WireCuts {
    uint32_t n;           // ranges, 1 .. 64
    uint32_t cut[65];     // cut[0] = 0 < cut[1] < ... < cut[n] = count
};

// A header at h: (L_t, the bits of M_t), each a little-endian uint32; with
// dword loads where h is 4-byte aligned (a later range's headers need not be)
__device__ __forceinline__ uint2 wire_hdr(const uint8_t* h) {
    if ((reinterpret_cast<uintptr_t>(h) & 3) == 0) {
        const uint32_t* const w = reinterpret_cast<const uint32_t*>(h);
        return make_uint2(w[0], w[1]);
    }
    uint32_t l = 0, m = 0;
#pragma unroll
    for (uint32_t b = 0; b < 4; ++b) {
        l |= (uint32_t)h[b] << (8 * b);
        m |= (uint32_t)h[4 + b] << (8 * b);
    }
    return make_uint2(l, m);
}

// One block over all tensors, kThreads * kWirePer per round, after (unpack)
// one wavefront has located each range's headers in order (it also resets
// *status, which only it raises): each stream's
// length (pack: from in_lens; unpack: from its header), checked against its
// slot (a longer one is TLC_ERR_CORRUPT and counts as empty); the headers
// (pack) or out_lens and scales (unpack); the exclusive prefix of the lengths
// (woff[t]: where stream t starts in the message body; woff[count]: their
// sum) and of their 4 KiB chunks (cfirst[t]); ctrl[0] = chunks; the message
// length (pack).  Unpack: messages shorter than their headers and streams are
// TLC_ERR_CORRUPT, and then no chunk is copied (the tensors whose headers were
// not in them get length 0 and M = 0).
template <bool kPack>
__global__ __launch_bounds__(kThreads) void k_wire_scan(GroupView g, WireCuts cuts, const uint64_t* __restrict__ lens_in,
                                                        const float* __restrict__ m_in, uint8_t* __restrict__ hdr_out,
                                                        const uint8_t* __restrict__ hdr_in, uint64_t wire_bytes,
                                                        uint64_t* __restrict__ lens_out, float* __restrict__ m_out,
                                                        uint64_t* __restrict__ woff, uint64_t* __restrict__ dbase,
                                                        uint32_t* __restrict__ cfirst, uint32_t* __restrict__ ctrl,
                                                        uint64_t* __restrict__ wire_len, int* __restrict__ status) {
    __shared__ uint64_t s_sm[kWaves];
    __shared__ uint32_t s_u[kWaves];
    __shared__ uint32_t s_cut[65];
    __shared__ uint64_t s_hbase[64];  // unpack: where range q's headers start
    const uint32_t count = g.count;
    if (threadIdx.x == 0) *status = TLC_OK;  // the call's only kernel that reports
    if (threadIdx.x <= cuts.n) s_cut[threadIdx.x] = cuts.cut[threadIdx.x];
    __syncthreads();
    uint64_t carry_b = 0;  // bytes of the rounds before
    uint32_t carry_c = 0;  // chunks of the rounds before
    bool bad = false;
    uint32_t read_to = count;  // tensors below it have their headers inside the messages
    if (!kPack) {
        // where each range's headers start: message q's headers follow the
        // bodies of the ranges before it, so one wavefront locates the ranges
        // in order, summing each range's lengths (a length above its slot
        // counts as 0, as below); a range whose headers run past wire_bytes
        // ends the walk
        __shared__ uint32_t s_readto;
        if (threadIdx.x < 64) {
            uint64_t hb = 0;  // the lengths of the ranges before
            uint32_t rt = count;
            for (uint32_t q = 0; q < cuts.n; ++q) {
                const uint32_t a = s_cut[q], z = s_cut[q + 1];
                const uint64_t base = 8ull * a + hb;
                if (base + 8ull * (z - a) > wire_bytes) {  // wave-uniform
                    rt = a;
                    break;
                }
                if (threadIdx.x == 0) s_hbase[q] = base;
                if (q + 1 == cuts.n) break;  // no range after it: its lengths are not needed here
                uint64_t sum = 0;
                for (uint32_t t = a + threadIdx.x; t < z; t += 64) {
                    const uint64_t l = wire_hdr(hdr_in + base + 8ull * (t - a)).x;
                    if (l <= quartic_len(load_seg(g, t).n)) sum += l;
                }
                for (int d = 32; d >= 1; d >>= 1) {
                    const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)sum, d, 64);
                    const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(sum >> 32), d, 64);
                    sum += (uint64_t)hi << 32 | lo;
                }
                hb += sum;
            }
            if (threadIdx.x == 0) s_readto = rt;
        }
        __syncthreads();
        read_to = s_readto;
    }
    // all tensors in rounds; a thread's tensors are consecutive, so its range
    // index only moves forward
    for (uint32_t r0 = 0; r0 < count; r0 += kThreads * kWirePer) {
        const uint32_t t0 = r0 + threadIdx.x * kWirePer;
        uint32_t L[kWirePer];
        uint64_t my_b = 0;
        uint32_t my_c = 0;
        uint32_t k = 0;
        if (!kPack && t0 < count) {
            uint32_t hi = cuts.n;  // s_cut[k] <= t0 < s_cut[hi]
            while (hi - k > 1) {
                const uint32_t mid = (k + hi) / 2;
                if (s_cut[mid] <= t0) k = mid;
                else hi = mid;
            }
        }
#pragma unroll
        for (int j = 0; j < (int)kWirePer; ++j) {
            const uint32_t t = t0 + (uint32_t)j;
            L[j] = 0;
            if (t < count) {
                const uint64_t cap = quartic_len(load_seg(g, t).n);
                uint64_t l = 0;
                uint32_t mb = 0;
                if (kPack) {
                    l = lens_in[t];
                    mb = __float_as_uint(m_in[t]);
                } else if (t < read_to) {
                    while (s_cut[k + 1] <= t) ++k;
                    const uint2 h = wire_hdr(hdr_in + s_hbase[k] + 8ull * (t - s_cut[k]));
                    l = h.x;
                    mb = h.y;
                }
                if (l > cap) {
                    bad = true;
                    l = 0;
                }
                if (!kPack) {
                    lens_out[t] = l;
                    m_out[t] = __uint_as_float(mb);
                }
                L[j] = (uint32_t)l;
                my_b += l;
                my_c += (uint32_t)((l + kWireChunk - 1) / kWireChunk);
            }
        }
        uint64_t tot_b;
        uint32_t tot_c;
        uint64_t b = carry_b + block_excl_scan(my_b, 0ull, SumCompose(), s_sm, &tot_b);
        uint32_t c = carry_c + block_excl_sum(my_c, s_u, &tot_c);
#pragma unroll
        for (int j = 0; j < (int)kWirePer; ++j) {
            const uint32_t t = t0 + (uint32_t)j;
            if (t < count) {
                woff[t] = b;
                cfirst[t] = c;
                b += L[j];
                c += (uint32_t)((L[j] + kWireChunk - 1) / kWireChunk);
            }
        }
        carry_b += tot_b;
        carry_c += tot_c;
    }
    if (__syncthreads_or(bad) && threadIdx.x == 0) raise_status(status, TLC_ERR_CORRUPT);
    if (threadIdx.x == 0) {
        woff[count] = carry_b;
        const uint64_t total = 8ull * count + carry_b;
        const bool fits = kPack || (read_to == count && total <= wire_bytes);
        if (!fits) raise_status(status, TLC_ERR_CORRUPT);
        ctrl[0] = fits ? carry_c : 0u;
    }
    __syncthreads();  // every woff entry written above is visible to the block
    // where each stream goes in the messages, and (pack) the headers and each
    // message's length: one tensor per thread and round, so that the rounds'
    // loads are independent; its range by a binary search over the cuts
    for (uint32_t u = threadIdx.x; u < count; u += kThreads) {
        uint32_t lo = 0, hi = cuts.n;  // s_cut[lo] <= u < s_cut[hi]
        while (hi - lo > 1) {
            const uint32_t mid = (lo + hi) / 2;
            if (s_cut[mid] <= u) lo = mid;
            else hi = mid;
        }
        const uint64_t wu = woff[u];
        dbase[u] = 8ull * s_cut[lo + 1] + wu;
        if (kPack) {  // byte stores: a later range's headers need not be 4-byte aligned
            uint8_t* const h = hdr_out + 8ull * u + woff[s_cut[lo]];
            const uint32_t l = (uint32_t)(woff[u + 1] - wu), mb = __float_as_uint(m_in[u]);
#pragma unroll
            for (uint32_t b = 0; b < 4; ++b) {
                h[b] = (uint8_t)(l >> (8 * b));
                h[4 + b] = (uint8_t)(mb >> (8 * b));
            }
        }
    }
    if (kPack && threadIdx.x < cuts.n) {
        const uint32_t a = s_cut[threadIdx.x], b = s_cut[threadIdx.x + 1];
        wire_len[threadIdx.x] = 8ull * (b - a) + woff[b] - woff[a];
    }
}

// 16 bytes of the LDS buffer from byte `off` (0 <= off, off + 16 <= its size)
__device__ __forceinline__ uint4 lds_bytes16(const uint32_t* buf, uint32_t off) {
    const uint32_t w = off >> 2, sh = 8u * (off & 3u);
    uint32_t d[5];
#pragma unroll
    for (int k = 0; k < 5; ++k) d[k] = buf[w + k];
    auto cut = [&](uint32_t lo, uint32_t hi) { return sh ? (lo >> sh) | (hi << (32u - sh)) : lo; };
    return make_uint4(cut(d[0], d[1]), cut(d[1], d[2]), cut(d[2], d[3]), cut(d[3], d[4]));
}

// Copies every stream's bytes between its slot and the message body, one
// 4 KiB chunk of one stream per block and round (the chunk's tensor by a
// binary search over cfirst, held in LDS when the group has at most 4096
// tensors).  The chunk goes through LDS so that the side
// the chunk is not 16-byte aligned on is read or written in whole aligned
// words: pack reads its slot (aligned) and writes the body, where a word that
// the chunk shares with a neighbour is written byte by byte; unpack reads the
// body with whole words only inside [0, wire_bytes), byte by byte past that,
// and writes its slot (aligned; the bytes after the stream in its last word
// are written as 0, still inside the slot).
template <bool kPack>
__global__ __launch_bounds__(kThreads) void k_wire_copy(GroupView g, const uint8_t* __restrict__ src,
                                                        uint8_t* __restrict__ dst, uint64_t wire_bytes,
                                                        const uint64_t* __restrict__ woff,
                                                        const uint64_t* __restrict__ dbase,
                                                        const uint32_t* __restrict__ cfirst,
                                                        const uint32_t* __restrict__ ctrl) {
    constexpr uint32_t kWireLdsTensors = 4096;  // groups up to this many tensors search their chunks in LDS
    __shared__ __align__(16) uint32_t s_buf[(kWireChunk + 32) / 4 + 8];
    __shared__ uint32_t s_cf[kWireLdsTensors];
    __shared__ uint32_t s_t;
    const uint32_t nchunks = ctrl[0];
    const uint32_t count = g.count;
    const uint32_t i = threadIdx.x;
    const bool in_lds = count <= kWireLdsTensors;
    if (blockIdx.x >= nchunks) return;
    if (in_lds) {
        for (uint32_t k = i; k < count; k += kThreads) s_cf[k] = cfirst[k];
        __syncthreads();
    }
    for (uint32_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
        if (i == 0) {  // the last tensor whose first chunk is <= c
            uint32_t lo = 0, hi = count;
            while (hi - lo > 1) {
                const uint32_t mid = (lo + hi) >> 1;
                if ((in_lds ? s_cf[mid] : cfirst[mid]) <= c) lo = mid;
                else hi = mid;
            }
            s_t = lo;
        }
        __syncthreads();
        const uint32_t t = s_t;
        const Seg sg = load_seg(g, t);
        const uint64_t k0 = (uint64_t)(c - cfirst[t]) * kWireChunk;  // first byte of the chunk in stream t
        const uint64_t L = woff[t + 1] - woff[t];
        const uint32_t len = (uint32_t)min<uint64_t>(kWireChunk, L - k0);
        const uint64_t slot = sg.stream_off + k0;   // aligned
        const uint64_t msg = dbase[t] + k0;         // any alignment
        if (kPack) {
            // slot words straight into LDS: data byte m at buffer byte m
            if (16u * i < len) reinterpret_cast<uint4*>(s_buf)[i] = reinterpret_cast<const uint4*>(src + slot)[i];
            __syncthreads();
            const uint32_t mis = (uint32_t)(msg & 15u);
            const uint64_t a0 = msg - mis;  // aligned word j covers data bytes 16 j - mis .. + 15
            const uint32_t nw = (mis + len + 15) / 16;  // up to 257
            for (uint32_t wi = i; wi < nw; wi += kThreads) {
                const int32_t m0 = 16 * (int32_t)wi - (int32_t)mis;
                if (m0 >= 0 && m0 + 16 <= (int32_t)len) {
                    *reinterpret_cast<uint4*>(dst + a0 + 16ull * wi) = lds_bytes16(s_buf, (uint32_t)m0);
                } else {
                    const uint8_t* const b8 = reinterpret_cast<const uint8_t*>(s_buf);
                    for (int32_t j = 0; j < 16; ++j) {
                        const int32_t m = m0 + j;
                        if (m >= 0 && m < (int32_t)len) dst[a0 + 16ull * wi + (uint32_t)j] = b8[m];
                    }
                }
            }
        } else {
            // body words into LDS: data byte m at buffer byte smis + m
            const uint32_t smis = (uint32_t)(msg & 15u);
            const uint64_t a0 = msg - smis;
            const uint32_t nw = (smis + len + 15) / 16;  // up to 257
            for (uint32_t wi = i; wi < nw; wi += kThreads) {
                const uint64_t w = a0 + 16ull * wi;
                uint4 v = make_uint4(0u, 0u, 0u, 0u);
                if (w + 16 <= wire_bytes) {
                    v = *reinterpret_cast<const uint4*>(src + w);
                } else {
                    uint32_t d[4] = {0u, 0u, 0u, 0u};
                    for (uint32_t j = 0; j < 16; ++j)
                        if (w + j < wire_bytes) d[j >> 2] |= (uint32_t)src[w + j] << (8u * (j & 3u));
                    v = make_uint4(d[0], d[1], d[2], d[3]);
                }
                reinterpret_cast<uint4*>(s_buf)[wi] = v;
            }
            __syncthreads();
            if (16u * i < len) {
                uint4 v = lds_bytes16(s_buf, smis + 16u * i);
                const uint32_t keep = min(16u, len - 16u * i);  // data bytes of this word
                if (keep < 16u) {
                    uint32_t* const d = reinterpret_cast<uint32_t*>(&v);
                    for (uint32_t j = 0; j < 4; ++j) {
                        const uint32_t b = keep > 4 * j ? min(4u, keep - 4 * j) : 0u;
                        d[j] &= b >= 4 ? ~0u : ((1u << (8 * b)) - 1u);
                    }
                }
                *reinterpret_cast<uint4*>(dst + slot + 16ull * i) = v;
            }
        }
        __syncthreads();  // s_buf and s_t are rewritten by the next chunk
    }
}

// ---------------------------------------------------------------------------
// host side

struct ProfRec {
    const char* name;
    hipEvent_t a, b;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
char g_prof_only[48] = {0};  // when set, only this kernel is bracketed
std::vector<ProfRec> g_prof;

template <typename Launch>
int launch(const char* name, hipStream_t st, Launch&& fn) {
    hipEvent_t a = nullptr, b = nullptr;
    bool prof;
    {
        std::lock_guard<std::mutex> lk(g_prof_mu);
        prof = g_prof_on && (!g_prof_only[0] || strcmp(g_prof_only, name) == 0);
    }
    if (prof) {
        if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) return TLC_ERR_HIP;
        if (hipEventRecord(a, st) != hipSuccess) return TLC_ERR_HIP;
    }
    fn();
    if (hipGetLastError() != hipSuccess) return TLC_ERR_HIP;
    if (prof) {
        if (hipEventRecord(b, st) != hipSuccess) return TLC_ERR_HIP;
        std::lock_guard<std::mutex> lk(g_prof_mu);
        g_prof.push_back({name, a, b});
    }
    return TLC_OK;
}

// Blocks of a grid-looping kernel that are resident on the current device at
// once (occupancy per CU times the CU count, at most `cap`), queried once per
// device.  Such kernels hand work to their blocks or waves round-robin, so a
// grid larger than this leaves a second, partial round of blocks running
// alone at the end.
enum GridKind {
    kGridPack, kGridDecodeWrite, kGridDecodeAdd, kGridDecodeRecord, kGridDecodeWide, kGridApply, kGridWirePack, kGridWireUnpack, kGridKinds
};
uint32_t resident_grid(GridKind kind, const void* kern, uint32_t cap, int threads = kThreads) {
    static std::mutex mu;
    static std::vector<uint32_t> per_dev;  // kGridKinds entries per device, 0 = not queried
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return cap;
    std::lock_guard<std::mutex> lk(mu);
    const size_t at = (size_t)dev * kGridKinds + kind;
    if (at >= per_dev.size()) per_dev.resize(at + 1, 0);
    if (!per_dev[at]) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, threads, 0) == hipSuccess && cus > 0 &&
            per_cu > 0)
            per_dev[at] = (uint32_t)std::min<int64_t>((int64_t)cus * per_cu, cap);
        else
            per_dev[at] = cap, (void)hipGetLastError();  // a failed query leaves no error behind
    }
    return per_dev[at];
}

constexpr size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

constexpr uint64_t ftiles_of(uint64_t total) { return (total + kFTile - 1) / kFTile; }
constexpr uint64_t etiles_host(uint64_t n) { return (n + kETile - 1) / kETile; }
constexpr uint64_t spans_host(uint64_t n) { return (etiles_host(n) + kSpan - 1) / kSpan; }
constexpr uint64_t chunks_host(uint64_t n) {
    return ((n + 4) / 5 + kChunk - 1) / kChunk > 1 ? ((n + 4) / 5 + kChunk - 1) / kChunk : 1;
}

// Sizes of everything a call needs, for one tensor or a group.
struct Dims {
    uint64_t count, total, ftiles, etiles, spans, chunks;
};

struct Layout {
    size_t ctrl = 0, pmax = 0, etile_agg = 0, etmax = 0, active = 0, mbits = 0, seg_cb = 0, cand_cnt = 0, cand = 0,
           span_flags = 0, span_tickets = 0, chunk_tickets = 0, staging = 0, dec_flags = 0, dec_map = 0,
           dec_first = 0, total = 0;
};

constexpr Layout ws_layout(const Dims& d) {
    Layout l;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align_up(off + bytes, 256);
        return at;
    };
    l.ctrl = take(256);
    l.pmax = take((d.ftiles + d.count) * sizeof(float));
    l.etile_agg = take(d.etiles * sizeof(uint64_t));
    l.etmax = take(d.etiles * sizeof(float));
    l.active = take(d.etiles * sizeof(PackJob));
    l.mbits = take(d.count * sizeof(uint32_t));
    l.seg_cb = take(d.count * sizeof(float));
    l.cand_cnt = take(d.ftiles * sizeof(uint16_t));
    l.cand = take(d.ftiles * kCand * sizeof(uint2));
    l.span_flags = take(d.spans * sizeof(uint64_t));
    l.span_tickets = take(d.count * sizeof(uint32_t));
    l.chunk_tickets = take(d.count * sizeof(uint32_t));
    l.staging = take(d.etiles * kETileBytes);
    l.dec_flags = take(d.chunks * sizeof(uint64_t));
    l.dec_map = take(d.chunks * sizeof(uint32_t));
    l.dec_first = take(d.count * sizeof(uint32_t));
    l.total = off;
    return l;
}

constexpr Dims single_dims(uint64_t n) { return {1, n, ftiles_of(n), etiles_host(n), spans_host(n), chunks_host(n)}; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
bool valid_s(float s) { return s >= 1.0f && s < 2.0f; }  // false for NaN

struct Plan {
    GroupView g;
    Dims d;
};

Plan single_plan(uint64_t n) {
    Plan p;
    memset(&p.g, 0, sizeof(p.g));
    p.g.count = 1;
    p.g.one.n = (uint32_t)n;
    p.d = single_dims(n);
    return p;
}

struct TableLayout {
    size_t segs, ftile_info, span_seg, etile_seg, total;
};
TableLayout table_layout(const Dims& d) {
    TableLayout t;
    t.segs = sizeof(TableHeader);
    t.ftile_info = align_up(t.segs + d.count * sizeof(Seg), 16);
    t.span_seg = align_up(t.ftile_info + d.ftiles * sizeof(uint32_t), 16);
    t.etile_seg = align_up(t.span_seg + d.spans * sizeof(uint32_t), 16);
    t.total = align_up(t.etile_seg + d.etiles * sizeof(uint32_t), 16);
    return t;
}

Dims dims_of(const tlc_group_info* info) {
    return {info->count, info->total_elems, ftiles_of(info->total_elems), info->tiles, info->spans, info->chunks};
}

int group_plan_of(const tlc_group_info* info, const void* d_table, Plan* p) {
    if (!info || !d_table || !aligned16(d_table) || info->count == 0 || info->count > 0x7FFFFFFFull)
        return TLC_ERR_INVALID_ARG;
    p->d = dims_of(info);
    const TableLayout t = table_layout(p->d);
    if (t.total != info->table_bytes || ws_layout(p->d).total != info->workspace_bytes) return TLC_ERR_INVALID_ARG;
    const char* base = static_cast<const char*>(d_table);
    memset(&p->g, 0, sizeof(p->g));
    p->g.segs = reinterpret_cast<const Seg*>(base + t.segs);
    p->g.ftile_info = reinterpret_cast<const uint32_t*>(base + t.ftile_info);
    p->g.span_seg = reinterpret_cast<const uint32_t*>(base + t.span_seg);
    p->g.etile_seg = reinterpret_cast<const uint32_t*>(base + t.etile_seg);
    p->g.count = (uint32_t)info->count;
    return TLC_OK;
}

int check_ws(const Plan& p, void* ws, size_t ws_bytes, Layout* l) {
    *l = ws_layout(p.d);
    if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255) || ws_bytes < l->total) return TLC_ERR_WORKSPACE;
    return TLC_OK;
}

// fo.enc == 0: the 3LC stream into out/out_lens; otherwise a fixed-length
// encoding into fo (out and out_lens unused)
int run_compress(const Plan& p, const float* x, float x_div, float* err, float s, uint8_t* out, uint64_t* out_lens,
                 float* scales, void* ws, size_t ws_bytes, int* status, hipStream_t st,
                 const FixedOut& fo = FixedOut{0, nullptr, nullptr}) {
    if (!x || !err || !scales || !status) return TLC_ERR_INVALID_ARG;
    if (fo.enc ? !fo.out : (!out || !out_lens)) return TLC_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(err) || !valid_s(s)) return TLC_ERR_INVALID_ARG;
    Layout l;
    int rc = check_ws(p, ws, ws_bytes, &l);
    if (rc) return rc;
    char* w = static_cast<char*>(ws);
    uint32_t* ctrl = reinterpret_cast<uint32_t*>(w + l.ctrl);
    float* pmax = reinterpret_cast<float*>(w + l.pmax);
    uint64_t* etile_agg = reinterpret_cast<uint64_t*>(w + l.etile_agg);
    float* etmax = reinterpret_cast<float*>(w + l.etmax);
    PackJob* jobs = reinterpret_cast<PackJob*>(w + l.active);
    uint32_t* mbits = reinterpret_cast<uint32_t*>(w + l.mbits);
    float* seg_cb = reinterpret_cast<float*>(w + l.seg_cb);
    uint16_t* cand_cnt = reinterpret_cast<uint16_t*>(w + l.cand_cnt);
    uint2* cand = reinterpret_cast<uint2*>(w + l.cand);
    uint64_t* span_flags = reinterpret_cast<uint64_t*>(w + l.span_flags);
    uint32_t* span_tickets = reinterpret_cast<uint32_t*>(w + l.span_tickets);
    uint8_t* staging = reinterpret_cast<uint8_t*>(w + l.staging);
    const GroupView g = p.g;
    const uint64_t N = p.d.total;
    const uint32_t ftiles = (uint32_t)p.d.ftiles, spans = (uint32_t)p.d.spans;
    const uint32_t pack_grid =
        (uint32_t)std::min<uint64_t>((p.d.etiles + kWaves - 1) / kWaves,
                                     resident_grid(kGridPack, reinterpret_cast<const void*>(k_quant_pack), kPackGrid));
    rc = launch("tlc_accum_max", st, [&] {
        k_accum_max<<<ftiles, kAccThreads, 0, st>>>(g, N, x, x_div, err, pmax, scales, s, cand_cnt, cand,
                                                 span_flags, p.d.spans, span_tickets, mbits, ctrl,
                                                 status);
    });
    if (rc) return rc;
    const uint32_t etiles = (uint32_t)p.d.etiles;
    rc = launch("tlc_tile_max", st, [&] {
        k_tile_max<<<(etiles + kThreads - 1) / kThreads, kThreads, 0, st>>>(g, etiles, pmax, etmax, mbits,
                                                                           scales, s, seg_cb);
    });
    if (rc) return rc;
    rc = launch("tlc_tile_activity", st, [&] {
        constexpr uint32_t per_block = kThreads * kActPerThread;
        k_tile_activity<<<(etiles + per_block - 1) / per_block, kThreads, 0, st>>>(g, etiles, s, pmax, etmax, mbits,
                                                                                 seg_cb, scales, etile_agg, jobs,
                                                                                 ctrl);
    });
    if (rc) return rc;
    if (fo.enc) {
        rc = launch("tlc_fixed_fill", st, [&] { k_fixed_fill<<<etiles, 64, 0, st>>>(g, etiles, fo); });
        if (rc) return rc;
    }
    rc = launch("tlc_quant_pack", st, [&] {
        k_quant_pack<<<pack_grid, kThreads, 0, st>>>(g, err, jobs, ctrl, etile_agg, staging, cand_cnt, cand, fo);
    });
    if (rc || fo.enc) return rc;
    return launch("tlc_emit", st, [&] {
        k_emit<<<spans, kThreads, 0, st>>>(g, etile_agg, staging, span_flags, span_tickets, out, out_lens, status);
    });
}

// Decoder state in a workspace: look-back flags and the chunk map for
// `payloads` payloads, per-unit ticket counters and first chunks; for the
// dense decompress and accumulate-many, each payload's tile starts and
// literal flags (one record of each per encode tile).
struct DecState {
    uint32_t* ctrl;
    uint64_t* flags;
    uint32_t* map;
    uint32_t* first;
    uint32_t* tickets;
    uint64_t* tstart;  // payload p's tile starts at tstart + p * etiles
    uint32_t* tlit;    // payload p's literal flags at tlit + p * etiles
};

// Decompress and the single-payload accumulate use the call's workspace:
// the compressor's per-tile summaries and maxima are not needed there, so
// their slots hold the tile starts and literal flags.
DecState dec_state_single(const Layout& l, char* w) {
    DecState d;
    d.ctrl = reinterpret_cast<uint32_t*>(w + l.ctrl);
    d.flags = reinterpret_cast<uint64_t*>(w + l.dec_flags);
    d.map = reinterpret_cast<uint32_t*>(w + l.dec_map);
    d.first = reinterpret_cast<uint32_t*>(w + l.dec_first);
    d.tickets = reinterpret_cast<uint32_t*>(w + l.chunk_tickets);
    d.tstart = reinterpret_cast<uint64_t*>(w + l.etile_agg);
    d.tlit = reinterpret_cast<uint32_t*>(w + l.etmax);
    return d;
}

// Whether P payloads of a group can be numbered: every (payload, tensor)
// unit id below the decoder's flag bit, every chunk number in 32 bits.
constexpr bool many_fits(const Dims& d, uint64_t P) {
    return P * d.count <= 0x7FFFFFFFull && P * d.chunks <= 0xFFFFFFFFull;
}

// Workspace of an accumulate-many call on P payloads.
struct ManyLayout {
    size_t ctrl = 0, flags = 0, map = 0, first = 0, tickets = 0, tstart = 0, tlit = 0, total = 0;
};
constexpr ManyLayout many_layout(const Dims& d, uint64_t P) {
    ManyLayout l;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align_up(off + bytes, 256);
        return at;
    };
    l.ctrl = take(256);
    l.flags = take(P * d.chunks * sizeof(uint64_t));
    l.map = take(P * d.chunks * sizeof(uint32_t));
    l.first = take(P * d.count * sizeof(uint32_t));
    l.tickets = take(P * d.count * sizeof(uint32_t));
    l.tstart = take(P * d.etiles * sizeof(uint64_t));
    l.tlit = take(P * d.etiles * sizeof(uint32_t));
    l.total = off;
    return l;
}

// k_prep for `payloads` payloads: n_fill: elements of y to zero first
// (sparse decompress); records: reset the tile records (record mode); hint:
// where the streams' density class goes (dense above dense_num / 1000
// stream bytes per quartic byte).
int launch_prep(const Plan& p, uint32_t payloads, bool records, uint32_t chunk, const uint64_t* in_lens, float* y,
                uint64_t n_fill, const DecState& ds, int* status, uint32_t* hint, uint32_t dense_num,
                hipStream_t st) {
    const GroupView g = p.g;
    const uint64_t chunks = p.d.chunks * payloads, etiles = p.d.etiles;
    uint64_t* const tstart = records ? ds.tstart : nullptr;
    const uint64_t ntiles = tstart ? payloads * etiles : 0;
    const uint64_t blocks = std::max((n_fill / 4 + kThreads - 1) / kThreads,
                                     (std::max(chunks, ntiles) + kThreads - 1) / kThreads);
    const uint32_t prep_grid = (uint32_t)std::min<uint64_t>(std::max<uint64_t>(blocks, 1), 1u << 20);
    return launch(n_fill ? "tlc_prep_fill" : "tlc_prep", st, [&] {
        if (n_fill)
            k_prep<true><<<prep_grid, kThreads, 0, st>>>(g, payloads, y, n_fill, in_lens, ds.flags, chunks, tstart,
                                                         ds.tlit, ntiles, ds.map, ds.first, ds.tickets, ds.ctrl,
                                                         status, hint, chunk, dense_num);
        else
            k_prep<false><<<prep_grid, kThreads, 0, st>>>(g, payloads, y, 0, in_lens, ds.flags, chunks, tstart,
                                                          ds.tlit, ntiles, ds.map, ds.first, ds.tickets, ds.ctrl,
                                                          status, hint, chunk, dense_num);
    });
}

// k_decode in `mode` over the chunks of units [u_lo, u_hi) of the last
// k_prep's set-up; `max_chunks` bounds their number (grid size).
int launch_dec(const Plan& p, int mode, bool wide, const uint8_t* in, uint64_t in_stride, const uint64_t* in_lens,
               const float* scales, float s, float* y, const DecState& ds, int* status, uint32_t u_lo, uint32_t u_hi,
               uint64_t max_chunks, hipStream_t st) {
    const GroupView g = p.g;
    const uint64_t etiles = p.d.etiles;
    uint64_t* const tstart = mode == kDecodeRecord ? ds.tstart : nullptr;
    auto kern = mode == kDecodeWrite ? k_decode<kDecodeWrite, 16>
                : mode == kDecodeAdd ? k_decode<kDecodeAdd, 16>
                : wide               ? k_decode<kDecodeRecord, kWideBPL>
                                     : k_decode<kDecodeRecord, 16>;
    const GridKind gk = wide ? kGridDecodeWide : (GridKind)(kGridDecodeWrite + mode);
    static const char* const names[] = {"tlc_decode", "tlc_decode_add", "tlc_decode_record"};
    const uint32_t grid = (uint32_t)std::min<uint64_t>(
        std::max<uint64_t>(max_chunks, 1), resident_grid(gk, reinterpret_cast<const void*>(kern), kDecodeGrid));
    return launch(wide ? "tlc_decode_record_wide" : names[mode], st, [&] {
        kern<<<grid, kThreads, 0, st>>>(g, in, in_stride, etiles, in_lens, scales, s, y, tstart, ds.tlit, ds.flags,
                                        ds.map, ds.first, ds.tickets, ds.ctrl, status, u_lo, u_hi);
    });
}

// k_prep, then k_decode in `mode` over the chunks of all `payloads` payloads.
// n_fill: elements of y to zero first (sparse decompress); hint: where the
// streams' density class goes, with the crossover dense_num / 1000.
int launch_decode(const Plan& p, uint32_t payloads, int mode, const uint8_t* in, uint64_t in_stride,
                  const uint64_t* in_lens, const float* scales, float s, float* y, uint64_t n_fill,
                  const DecState& ds, int* status, uint32_t* hint, uint32_t dense_num, hipStream_t st) {
    // the record pass over several payloads walks 16 KiB chunks (fewer
    // rounds of the resident grid); every other pass 4 KiB ones
    const bool wide = mode == kDecodeRecord && payloads > 1;
    const uint32_t chunk = wide ? kThreads * kWideBPL : kChunk;
    int rc = launch_prep(p, payloads, mode == kDecodeRecord, chunk, in_lens, y, n_fill, ds, status, hint, dense_num,
                         st);
    if (rc) return rc;
    return launch_dec(p, mode, wide, in, in_stride, in_lens, scales, s, y, ds, status, 0u, kToEnd,
                      p.d.chunks * payloads, st);
}

// Decompress takes one of two launch sequences, both giving the same y.
// Sparse: k_prep zero-fills y, then k_decode writes the nonzero codes over
// the fill.  Dense: k_decode records where each encode tile begins and
// k_expand writes every tile once.  The sparse path is faster while few tiles
// hold a nonzero code (the fill is the fastest way to write y, and few lines
// are written twice); the dense path once most tiles do (the scattered writes
// then land on lines the fill has already written).  The host cannot see the
// stream lengths without a synchronisation, so it follows the caller's hint
// word (host memory the device can write): the density class the previous
// decompress given the same word left there.  No word: the sparse path.
int run_decompress(const Plan& p, const uint8_t* in, const uint64_t* in_lens, const float* scales, float s,
                   float* y, void* ws, size_t ws_bytes, int* status, uint32_t* hint, uint32_t* dev_hint,
                   hipStream_t st, int accumulate) {
    if (!in || !in_lens || !scales || !y || !status) return TLC_ERR_INVALID_ARG;
    if (!aligned16(y) || !valid_s(s)) return TLC_ERR_INVALID_ARG;
    Layout l;
    int rc = check_ws(p, ws, ws_bytes, &l);
    if (rc) return rc;
    const DecState ds = dec_state_single(l, static_cast<char*>(ws));
    if (accumulate)
        return launch_decode(p, 1, kDecodeAdd, in, 0, in_lens, scales, s, y, 0, ds, status, nullptr,
                             (uint32_t)kDenseNum, st);
    const bool dense = hint && reinterpret_cast<volatile uint32_t*>(hint)[0] != 0u;
    rc = launch_decode(p, 1, dense ? kDecodeRecord : kDecodeWrite, in, 0, in_lens, scales, s, y,
                       dense ? 0 : p.d.total, ds, status, dev_hint, (uint32_t)kDenseNum, st);
    if (rc || !dense) return rc;
    const GroupView g = p.g;
    const uint64_t etiles = p.d.etiles;
    return launch("tlc_expand", st, [&] {
        k_expand<<<xcd_grid((etiles + kWaves - 1) / kWaves), kThreads, 0, st>>>(g, (uint32_t)etiles, in, in_lens,
                                                                                 scales, s, ds.tstart, ds.tlit, y,
                                                                                 status);
    });
}

// Accumulate-many takes one of two launch sequences, both giving the same
// acc.  Dense (no hint word, or a word holding 1): the tile starts of every
// payload in one decoder launch, then one pass over acc that decodes and
// applies them tile by tile.  Sparse (a word holding 0): one set-up for all
// payloads, then one add-mode decoder launch per payload in payload order,
// each touching only the elements its literal codes land on; while few tiles
// hold a nonzero code this moves far fewer bytes than a pass over every tile
// that any payload touches.  k_prep writes the density class of all the
// payloads' streams into the word.  stream_bytes: the group's stream buffer
// size (a payload's slots).
int run_accumulate_many(const Plan& p, uint64_t stream_bytes, uint32_t payloads, const uint8_t* in,
                        uint64_t in_stride, const uint64_t* in_lens, const float* scales, float s, float* acc,
                        void* ws, size_t ws_bytes, int* status, uint32_t* hint, uint32_t* dev_hint,
                        hipStream_t st) {
    if (!in || !in_lens || !scales || !acc || !status) return TLC_ERR_INVALID_ARG;
    if (payloads == 0 || payloads > kMaxPayloads || !aligned16(acc) || !valid_s(s)) return TLC_ERR_INVALID_ARG;
    if (!many_fits(p.d, payloads)) return TLC_ERR_TOO_LARGE;
    if (payloads > 1 && (in_stride < stream_bytes || (in_stride & 15))) return TLC_ERR_INVALID_ARG;
    const ManyLayout ml = many_layout(p.d, payloads);
    if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255) || ws_bytes < ml.total) return TLC_ERR_WORKSPACE;
    char* w = static_cast<char*>(ws);
    DecState ds;
    ds.ctrl = reinterpret_cast<uint32_t*>(w + ml.ctrl);
    ds.flags = reinterpret_cast<uint64_t*>(w + ml.flags);
    ds.map = reinterpret_cast<uint32_t*>(w + ml.map);
    ds.first = reinterpret_cast<uint32_t*>(w + ml.first);
    ds.tickets = reinterpret_cast<uint32_t*>(w + ml.tickets);
    ds.tstart = reinterpret_cast<uint64_t*>(w + ml.tstart);
    ds.tlit = reinterpret_cast<uint32_t*>(w + ml.tlit);
    const bool sparse = hint && reinterpret_cast<volatile uint32_t*>(hint)[0] == 0u;
    if (sparse) {
        int rc = launch_prep(p, payloads, false, kChunk, in_lens, nullptr, 0, ds, status, dev_hint,
                             (uint32_t)kManyDenseNum, st);
        for (uint32_t q = 0; q < payloads && !rc; ++q)
            rc = launch_dec(p, kDecodeAdd, false, in, in_stride, in_lens, scales, s, acc, ds, status,
                            q * (uint32_t)p.d.count, q + 1 < payloads ? (q + 1) * (uint32_t)p.d.count : kToEnd,
                            p.d.chunks, st);
        return rc;
    }
    int rc = launch_decode(p, payloads, kDecodeRecord, in, in_stride, in_lens, scales, s, nullptr, 0, ds, status,
                           dev_hint, (uint32_t)kManyDenseNum, st);
    if (rc) return rc;
    const GroupView g = p.g;
    const uint64_t etiles = p.d.etiles;
    const uint32_t nwaves = (uint32_t)std::min<uint64_t>(
        etiles, resident_grid(kGridApply, reinterpret_cast<const void*>(k_apply), 1u << 16, 64));
    return launch("tlc_apply", st, [&] {
        k_apply<<<xcd_grid(nwaves), 64, 0, st>>>(g, (uint32_t)etiles, nwaves, payloads, in, in_stride, in_lens,
                                                scales, s, ds.tstart, ds.tlit, acc, status);
    });
}

int run_decompress_fixed(const Plan& p, int enc, const uint8_t* in, const uint64_t* offs, const float* scales,
                         float s, float* y, int* status, hipStream_t st) {
    if (!in || !scales || !y || !status) return TLC_ERR_INVALID_ARG;
    if (!aligned16(y) || !valid_s(s)) return TLC_ERR_INVALID_ARG;
    int rc = launch("tlc_status_ok", st, [&] { k_status_ok<<<1, 1, 0, st>>>(status); });
    if (rc) return rc;
    return launch("tlc_fixed_decode", st, [&] {
        k_fixed_decode<<<xcd_grid((p.d.etiles + kWaves - 1) / kWaves), kThreads, 0, st>>>(
            p.g, (uint32_t)p.d.etiles, enc, in, offs, scales, s, y, status);
    });
}

bool valid_enc(int enc) { return enc == TLC_ENC_QUARTIC || enc == TLC_ENC_TWOBIT; }

// Compress without a caller workspace (tlc_compress_static): its scratch is a
// fixed device array of the workspace size of the largest tensor it takes.
// Each device holds its own copy from the first use until the process ends;
// host code reaches it only through the address hipGetSymbolAddress returns
// on that device (the array's name is not a device address on the host).
constexpr uint64_t kStaticMaxN = 1ull << 24;
constexpr size_t kStaticScratchBytes = ws_layout(single_dims(kStaticMaxN)).total;
static_assert(kStaticScratchBytes % 256 == 0 && kStaticScratchBytes < (32u << 20), "scratch size");
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

// The current device's address of `scratch`, looked up once per device (a
// symbol query, not an allocation); nullptr if the query fails.
void* static_scratch() {
    static std::mutex mu;
    static std::vector<void*> per_dev;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return nullptr;
    }
    std::lock_guard<std::mutex> lk(mu);
    if ((size_t)dev >= per_dev.size()) per_dev.resize(dev + 1, nullptr);
    if (!per_dev[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return nullptr;
        }
        per_dev[dev] = ptr;
    }
    return per_dev[dev];
}

int run_planes(bool gather, const float* src, const uint64_t* src_off, float* dst, const uint64_t* dst_off,
               const uint64_t* n, uint32_t count, uint64_t max_n, hipStream_t st) {
    if (!src || !src_off || !dst || !dst_off || !n || count == 0 || count > 65535 || max_n == 0 || max_n > kMaxN)
        return TLC_ERR_INVALID_ARG;  // one grid row per tensor: at most 65535
    const uint64_t bmax = (max_n + 4) / 5;  // byte positions of the largest tensor
    const dim3 grid((uint32_t)std::min<uint64_t>((bmax + kThreads - 1) / kThreads, 256), count);
    return launch(gather ? "tlc_planes_gather" : "tlc_planes_scatter", st, [&] {
        if (gather)
            k_planes<true><<<grid, kThreads, 0, st>>>(src, src_off, dst, dst_off, n);
        else
            k_planes<false><<<grid, kThreads, 0, st>>>(src, src_off, dst, dst_off, n);
    });
}
}  // namespace

// ---------------------------------------------------------------------------
// C ABI

// Workspace of the wire pack and unpack: the prefix of the stream lengths
// (count + 1), each stream's place in the messages, its first chunk, the
// chunk count.
struct WireLayout {
    size_t woff, dbase, cfirst, ctrl, total;
};
WireLayout wire_layout(uint64_t count) {
    WireLayout l;
    l.woff = 0;
    l.dbase = align_up(8 * (count + 1), 256);
    l.cfirst = l.dbase + align_up(8 * count, 256);
    l.ctrl = l.cfirst + align_up(4 * count, 256);
    l.total = l.ctrl + 256;
    return l;
}

// Host ranges -> kernel argument: cuts[0] = 0 < ... < cuts[n] = count, n <= 64.
bool wire_cuts(const uint32_t* cuts, uint32_t n, uint64_t count, WireCuts* wc) {
    if (n == 0 || n > 64) return false;
    if (!cuts) {
        if (n != 1) return false;
        wc->n = 1;
        wc->cut[0] = 0;
        wc->cut[1] = (uint32_t)count;
        return true;
    }
    if (cuts[0] != 0 || cuts[n] != count) return false;
    for (uint32_t k = 0; k < n; ++k)
        if (cuts[k] >= cuts[k + 1]) return false;
    wc->n = n;
    for (uint32_t k = 0; k <= n; ++k) wc->cut[k] = cuts[k];
    return true;
}

int run_wire(bool pack, const Plan& p, uint64_t stream_bytes, const uint32_t* cuts, uint32_t ranges,
             const uint8_t* slots_in, const uint64_t* lens_in, const float* m_in,
             uint8_t* wire, uint64_t wire_bytes, uint64_t* wire_len, const uint8_t* wire_in, uint8_t* slots_out,
             uint64_t* lens_out, float* m_out, void* ws, size_t ws_bytes, int* status, hipStream_t st) {
    const uint64_t count = p.d.count;
    if (!status) return TLC_ERR_INVALID_ARG;
    WireCuts wc;
    if (!wire_cuts(cuts, ranges, count, &wc)) return TLC_ERR_INVALID_ARG;
    if (pack) {
        if (!slots_in || !lens_in || !m_in || !wire || !wire_len || !aligned16(slots_in) || !aligned16(wire))
            return TLC_ERR_INVALID_ARG;
        if (wire_bytes < 8 * count + stream_bytes) return TLC_ERR_CAPACITY;
    } else {
        if (!wire_in || !slots_out || !lens_out || !m_out || !aligned16(wire_in) || !aligned16(slots_out))
            return TLC_ERR_INVALID_ARG;
        if (wire_bytes < 8 * count) return TLC_ERR_CAPACITY;
    }
    const WireLayout l = wire_layout(count);
    if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255) || ws_bytes < l.total) return TLC_ERR_WORKSPACE;
    char* const w = static_cast<char*>(ws);
    uint64_t* const woff = reinterpret_cast<uint64_t*>(w + l.woff);
    uint64_t* const dbase = reinterpret_cast<uint64_t*>(w + l.dbase);
    uint32_t* const cfirst = reinterpret_cast<uint32_t*>(w + l.cfirst);
    uint32_t* const ctrl = reinterpret_cast<uint32_t*>(w + l.ctrl);
    const GroupView g = p.g;
    int rc;
    const uint64_t chunk_bound = stream_bytes / kWireChunk + count;
    if (pack) {
        rc = launch("tlc_wire_scan", st, [&] {
            k_wire_scan<true><<<1, kThreads, 0, st>>>(g, wc, lens_in, m_in, wire, nullptr, 0, nullptr, nullptr, woff,
                                                      dbase, cfirst, ctrl, wire_len, status);
        });
        if (rc) return rc;
        const uint32_t grid = (uint32_t)std::min<uint64_t>(
            chunk_bound, resident_grid(kGridWirePack, reinterpret_cast<const void*>(k_wire_copy<true>), 1u << 16));
        return launch("tlc_wire_pack", st, [&] {
            k_wire_copy<true><<<grid, kThreads, 0, st>>>(g, slots_in, wire, wire_bytes, woff, dbase, cfirst, ctrl);
        });
    }
    rc = launch("tlc_wire_scan", st, [&] {
        k_wire_scan<false><<<1, kThreads, 0, st>>>(g, wc, nullptr, nullptr, nullptr, wire_in, wire_bytes, lens_out,
                                                   m_out, woff, dbase, cfirst, ctrl, nullptr, status);
    });
    if (rc) return rc;
    const uint32_t grid = (uint32_t)std::min<uint64_t>(
        chunk_bound, resident_grid(kGridWireUnpack, reinterpret_cast<const void*>(k_wire_copy<false>), 1u << 16));
    return launch("tlc_wire_unpack", st, [&] {
        k_wire_copy<false><<<grid, kThreads, 0, st>>>(g, wire_in, slots_out, wire_bytes, woff, dbase, cfirst, ctrl);
    });
}

extern "C" {

const char* tlc_status_string(int code) {
    switch (code) {
        case TLC_OK: return "ok";
        case TLC_ERR_INVALID_ARG: return "invalid argument";
        case TLC_ERR_CAPACITY: return "output capacity too small";
        case TLC_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case TLC_ERR_HIP: return "HIP runtime error";
        case TLC_ERR_CORRUPT: return "corrupt stream";
        case TLC_ERR_INTERNAL: return "internal wait expired";
        case TLC_ERR_TOO_LARGE: return "n above the largest tensor tlc_compress_static takes";
        default: return "unknown status";
    }
}

const char* tlc_version(void) { return "tlc-gfx950 0.2"; }

uint64_t tlc_compress_bound(uint64_t n) { return (n + 4) / 5; }

size_t tlc_workspace_size(uint64_t n) {
    if (n == 0 || n > kMaxN) return 0;
    return ws_layout(single_dims(n)).total;
}

int tlc_compress(const float* x, float* err, uint64_t n, float s, uint8_t* out, uint64_t out_capacity,
                 uint64_t* out_len, float* scale, void* workspace, size_t workspace_bytes, int* status,
                 tlc_stream_t stream) {
    if (n == 0 || n > kMaxN) return TLC_ERR_INVALID_ARG;
    if (out_capacity < tlc_compress_bound(n)) return TLC_ERR_CAPACITY;
    return run_compress(single_plan(n), x, 1.0f, err, s, out, out_len, scale, workspace, workspace_bytes, status,
                        static_cast<hipStream_t>(stream));
}

uint64_t tlc_compress_static_max_n(void) { return kStaticMaxN; }

int tlc_compress_static(const float* x, float* err, uint64_t n, float s, uint8_t* out, uint64_t out_capacity,
                        uint64_t* out_len, float* scale, int* status, tlc_stream_t stream) {
    if (n == 0) return TLC_ERR_INVALID_ARG;
    if (n > kStaticMaxN) return TLC_ERR_TOO_LARGE;
    if (out_capacity < tlc_compress_bound(n)) return TLC_ERR_CAPACITY;
    void* ws = static_scratch();
    if (!ws) return TLC_ERR_HIP;
    return run_compress(single_plan(n), x, 1.0f, err, s, out, out_len, scale, ws, kStaticScratchBytes, status,
                        static_cast<hipStream_t>(stream));
}

uint64_t tlc_fixed_len(uint64_t n, int encoding) {
    if (n == 0 || n > kMaxN || !valid_enc(encoding)) return 0;
    return fixed_len_of(n, encoding);
}

int tlc_compress_fixed(const float* x, float* err, uint64_t n, float s, int encoding, uint8_t* out,
                       uint64_t out_capacity, float* scale, void* workspace, size_t workspace_bytes, int* status,
                       tlc_stream_t stream) {
    if (n == 0 || n > kMaxN || !valid_enc(encoding)) return TLC_ERR_INVALID_ARG;
    if (out_capacity < fixed_len_of(n, encoding)) return TLC_ERR_CAPACITY;
    return run_compress(single_plan(n), x, 1.0f, err, s, nullptr, nullptr, scale, workspace, workspace_bytes, status,
                        static_cast<hipStream_t>(stream), FixedOut{encoding, out, nullptr});
}

int tlc_decompress_fixed(const uint8_t* in, const float* scale, uint64_t n, float s, int encoding, float* y,
                         int* status, tlc_stream_t stream) {
    if (n == 0 || n > kMaxN || !valid_enc(encoding)) return TLC_ERR_INVALID_ARG;
    return run_decompress_fixed(single_plan(n), encoding, in, nullptr, scale, s, y, status,
                                static_cast<hipStream_t>(stream));
}

int tlc_server_compress(const float* acc, uint32_t workers, float* err, uint64_t n, float s, uint8_t* out,
                        uint64_t out_capacity, uint64_t* out_len, float* scale, void* workspace,
                        size_t workspace_bytes, int* status, tlc_stream_t stream) {
    if (n == 0 || n > kMaxN || workers == 0) return TLC_ERR_INVALID_ARG;
    if (out_capacity < tlc_compress_bound(n)) return TLC_ERR_CAPACITY;
    return run_compress(single_plan(n), acc, (float)workers, err, s, out, out_len, scale, workspace,
                        workspace_bytes, status, static_cast<hipStream_t>(stream));
}

// The device address of the caller's hint word (pinned host memory), or
// nullptr; false if the word is not memory the device can reach.
bool hint_word(uint32_t* host, uint32_t** dev) {
    *dev = nullptr;
    if (!host) return true;
    void* d = nullptr;
    if (hipHostGetDevicePointer(&d, host, 0) != hipSuccess || !d) {
        (void)hipGetLastError();
        return false;
    }
    *dev = static_cast<uint32_t*>(d);
    return true;
}

int tlc_decompress(const uint8_t* in, const uint64_t* in_len, const float* scale, uint64_t n, float s, float* y,
                   void* workspace, size_t workspace_bytes, int* status, uint32_t* path_hint, tlc_stream_t stream) {
    if (n == 0 || n > kMaxN) return TLC_ERR_INVALID_ARG;
    uint32_t* dev_hint;
    if (!hint_word(path_hint, &dev_hint)) return TLC_ERR_INVALID_ARG;
    return run_decompress(single_plan(n), in, in_len, scale, s, y, workspace, workspace_bytes, status, path_hint,
                          dev_hint, static_cast<hipStream_t>(stream), 0);
}

int tlc_decompress_accumulate(const uint8_t* in, const uint64_t* in_len, const float* scale, uint64_t n, float s,
                              float* acc, void* workspace, size_t workspace_bytes, int* status,
                              tlc_stream_t stream) {
    if (n == 0 || n > kMaxN) return TLC_ERR_INVALID_ARG;
    return run_decompress(single_plan(n), in, in_len, scale, s, acc, workspace, workspace_bytes, status, nullptr,
                          nullptr, static_cast<hipStream_t>(stream), 1);
}

int tlc_group_plan(const uint64_t* sizes, uint64_t count, tlc_group_info* info, void* table,
                   size_t table_capacity, uint64_t* stream_offset) {
    if (!sizes || !info || count == 0 || count > 0x7FFFFFFFull) return TLC_ERR_INVALID_ARG;
    Dims d = {count, 0, 0, 0, 0, 0};
    uint64_t stream = 0;
    for (uint64_t i = 0; i < count; ++i) {
        const uint64_t n = sizes[i];
        if (n == 0 || n > kMaxN) return TLC_ERR_INVALID_ARG;
        d.total += n;
        d.etiles += etiles_host(n);
        d.spans += spans_host(n);
        d.chunks += chunks_host(n);
        stream = align_up(stream, 16) + tlc_compress_bound(n);
    }
    d.ftiles = ftiles_of(d.total);
    if (d.ftiles + d.count > 0xFFFFFFFFull || d.etiles > 0xFFFFFFFFull || d.chunks > 0xFFFFFFFFull)
        return TLC_ERR_INVALID_ARG;
    const TableLayout t = table_layout(d);
    info->count = count;
    info->total_elems = d.total;
    info->stream_bytes = align_up(stream, 16);
    info->table_bytes = t.total;
    info->workspace_bytes = ws_layout(d).total;
    info->tiles = d.etiles;
    info->chunks = d.chunks;
    info->spans = d.spans;
    if (!table && !stream_offset) return TLC_OK;
    if (table && table_capacity < t.total) return TLC_ERR_CAPACITY;
    char* base = static_cast<char*>(table);
    uint32_t* ftile_info = table ? reinterpret_cast<uint32_t*>(base + t.ftile_info) : nullptr;
    uint32_t* span_seg = table ? reinterpret_cast<uint32_t*>(base + t.span_seg) : nullptr;
    uint32_t* etile_seg = table ? reinterpret_cast<uint32_t*>(base + t.etile_seg) : nullptr;
    if (table) {
        memset(base, 0, t.total);
        TableHeader h = {kMagic, count, d.ftiles, d.etiles, d.spans, d.chunks, d.total, info->stream_bytes};
        memcpy(base, &h, sizeof(h));
    }
    uint64_t etile = 0, span = 0, chunk = 0, eoff = 0, soff = 0, ft = 0;
    for (uint64_t i = 0; i < count; ++i) {
        const uint64_t n = sizes[i];
        soff = align_up(soff, 16);
        if (stream_offset) stream_offset[i] = soff;
        if (table) {
            Seg sg;
            sg.elem_off = eoff;
            sg.n = (uint32_t)n;
            sg.etile0 = (uint32_t)etile;
            sg.stream_off = soff;
            sg.span0 = (uint32_t)span;
            sg.chunk0 = (uint32_t)chunk;
            memcpy(base + t.segs + i * sizeof(Seg), &sg, sizeof(Seg));
            for (uint64_t k = 0; k < spans_host(n); ++k) span_seg[span + k] = (uint32_t)i | (spans_host(n) > 1 ? kMulti : 0u);
            for (uint64_t k = 0; k < etiles_host(n); ++k) etile_seg[etile + k] = (uint32_t)i;
            // flat tiles whose first element lies in this tensor
            const uint64_t end = eoff + n;
            for (; ft < d.ftiles && ft * kFTile < end; ++ft) {
                const uint64_t last = std::min<uint64_t>(d.total, (ft + 1) * kFTile) - 1;
                ftile_info[ft] = (uint32_t)i | (last >= end ? kStraddle : 0u);
            }
        }
        etile += etiles_host(n);
        span += spans_host(n);
        chunk += chunks_host(n);
        eoff += n;
        soff += tlc_compress_bound(n);
    }
    return TLC_OK;
}

int tlc_compress_group(const tlc_group_info* info, const void* d_table, const float* x, float* err, float s,
                       uint8_t* out, uint64_t* out_lens, float* scales, void* workspace, size_t workspace_bytes,
                       int* status, tlc_stream_t stream) {
    Plan p;
    int rc = group_plan_of(info, d_table, &p);
    if (rc) return rc;
    return run_compress(p, x, 1.0f, err, s, out, out_lens, scales, workspace, workspace_bytes, status,
                        static_cast<hipStream_t>(stream));
}

int tlc_compress_fixed_group(const tlc_group_info* info, const void* d_table, int encoding, const float* x,
                             float* err, float s, uint8_t* out, const uint64_t* out_offsets, float* scales,
                             void* workspace, size_t workspace_bytes, int* status, tlc_stream_t stream) {
    if (!valid_enc(encoding) || !out_offsets) return TLC_ERR_INVALID_ARG;
    Plan p;
    int rc = group_plan_of(info, d_table, &p);
    if (rc) return rc;
    return run_compress(p, x, 1.0f, err, s, nullptr, nullptr, scales, workspace, workspace_bytes, status,
                        static_cast<hipStream_t>(stream), FixedOut{encoding, out, out_offsets});
}

int tlc_decompress_fixed_group(const tlc_group_info* info, const void* d_table, int encoding, const uint8_t* in,
                               const uint64_t* in_offsets, const float* scales, float s, float* y, int* status,
                               tlc_stream_t stream) {
    if (!valid_enc(encoding) || !in_offsets) return TLC_ERR_INVALID_ARG;
    Plan p;
    int rc = group_plan_of(info, d_table, &p);
    if (rc) return rc;
    return run_decompress_fixed(p, encoding, in, in_offsets, scales, s, y, status, static_cast<hipStream_t>(stream));
}

int tlc_server_compress_group(const tlc_group_info* info, const void* d_table, const float* acc, uint32_t workers,
                              float* err, float s, uint8_t* out, uint64_t* out_lens, float* scales, void* workspace,
                              size_t workspace_bytes, int* status, tlc_stream_t stream) {
    if (workers == 0) return TLC_ERR_INVALID_ARG;
    Plan p;
    int rc = group_plan_of(info, d_table, &p);
    if (rc) return rc;
    return run_compress(p, acc, (float)workers, err, s, out, out_lens, scales, workspace, workspace_bytes, status,
                        static_cast<hipStream_t>(stream));
}

int tlc_decompress_group(const tlc_group_info* info, const void* d_table, const uint8_t* in,
                         const uint64_t* in_lens, const float* scales, float s, float* y, void* workspace,
                         size_t workspace_bytes, int* status, uint32_t* path_hint, tlc_stream_t stream) {
    Plan p;
    int rc = group_plan_of(info, d_table, &p);
    if (rc) return rc;
    uint32_t* dev_hint;
    if (!hint_word(path_hint, &dev_hint)) return TLC_ERR_INVALID_ARG;
    return run_decompress(p, in, in_lens, scales, s, y, workspace, workspace_bytes, status, path_hint, dev_hint,
                          static_cast<hipStream_t>(stream), 0);
}

int tlc_decompress_accumulate_group(const tlc_group_info* info, const void* d_table, const uint8_t* in,
                                    const uint64_t* in_lens, const float* scales, float s, float* acc,
                                    void* workspace, size_t workspace_bytes, int* status, tlc_stream_t stream) {
    Plan p;
    int rc = group_plan_of(info, d_table, &p);
    if (rc) return rc;
    return run_decompress(p, in, in_lens, scales, s, acc, workspace, workspace_bytes, status, nullptr, nullptr,
                          static_cast<hipStream_t>(stream), 1);
}

uint64_t tlc_wire_bound(const tlc_group_info* info) {
    if (!info || info->count == 0) return 0;
    return 8 * info->count + info->stream_bytes;
}

uint64_t tlc_wire_workspace_size(const tlc_group_info* info) {
    if (!info || info->count == 0) return 0;
    return wire_layout(info->count).total;
}

int tlc_wire_pack_group(const tlc_group_info* info, const void* d_table, const uint8_t* in, const uint64_t* in_lens,
                        const float* scales, uint8_t* wire, uint64_t wire_capacity, uint64_t* wire_len,
                        void* workspace, size_t workspace_bytes, int* status, tlc_stream_t stream) {
    Plan p;
    int rc = group_plan_of(info, d_table, &p);
    if (rc) return rc;
    return run_wire(true, p, info->stream_bytes, nullptr, 1, in, in_lens, scales, wire, wire_capacity, wire_len, nullptr, nullptr, nullptr, nullptr,
                    workspace, workspace_bytes, status, static_cast<hipStream_t>(stream));
}

int tlc_wire_pack_ranges_group(const tlc_group_info* info, const void* d_table, const uint32_t* cuts, uint32_t ranges,
                               const uint8_t* in, const uint64_t* in_lens, const float* scales, uint8_t* wire,
                               uint64_t wire_capacity, uint64_t* wire_lens, void* workspace, size_t workspace_bytes,
                               int* status, tlc_stream_t stream) {
    Plan p;
    int rc = group_plan_of(info, d_table, &p);
    if (rc) return rc;
    if (!cuts) return TLC_ERR_INVALID_ARG;
    return run_wire(true, p, info->stream_bytes, cuts, ranges, in, in_lens, scales, wire, wire_capacity, wire_lens,
                    nullptr, nullptr, nullptr, nullptr, workspace, workspace_bytes, status,
                    static_cast<hipStream_t>(stream));
}

int tlc_wire_unpack_ranges_group(const tlc_group_info* info, const void* d_table, const uint32_t* cuts,
                                 uint32_t ranges, const uint8_t* wire, uint64_t wire_bytes, uint8_t* out,
                                 uint64_t* out_lens, float* scales, void* workspace, size_t workspace_bytes,
                                 int* status, tlc_stream_t stream) {
    Plan p;
    int rc = group_plan_of(info, d_table, &p);
    if (rc) return rc;
    if (!cuts) return TLC_ERR_INVALID_ARG;
    return run_wire(false, p, info->stream_bytes, cuts, ranges, nullptr, nullptr, nullptr, nullptr, wire_bytes,
                    nullptr, wire, out, out_lens, scales, workspace, workspace_bytes, status,
                    static_cast<hipStream_t>(stream));
}

int tlc_wire_unpack_group(const tlc_group_info* info, const void* d_table, const uint8_t* wire, uint64_t wire_bytes,
                          uint8_t* out, uint64_t* out_lens, float* scales, void* workspace, size_t workspace_bytes,
                          int* status, tlc_stream_t stream) {
    Plan p;
    int rc = group_plan_of(info, d_table, &p);
    if (rc) return rc;
    return run_wire(false, p, info->stream_bytes, nullptr, 1, nullptr, nullptr, nullptr, nullptr, wire_bytes, nullptr, wire, out, out_lens, scales,
                    workspace, workspace_bytes, status, static_cast<hipStream_t>(stream));
}

uint64_t tlc_accumulate_many_workspace_size(const tlc_group_info* info, uint32_t payloads) {
    if (!info || info->count == 0 || payloads == 0 || payloads > kMaxPayloads) return 0;
    const Dims d = dims_of(info);
    return many_fits(d, payloads) ? many_layout(d, payloads).total : 0;
}

int tlc_decompress_accumulate_many_group(const tlc_group_info* info, const void* d_table, uint32_t payloads,
                                         const uint8_t* in, uint64_t in_stride, const uint64_t* in_lens,
                                         const float* scales, float s, float* acc, void* workspace,
                                         size_t workspace_bytes, int* status, uint32_t* path_hint,
                                         tlc_stream_t stream) {
    Plan p;
    int rc = group_plan_of(info, d_table, &p);
    if (rc) return rc;
    uint32_t* dev_hint;
    if (!hint_word(path_hint, &dev_hint)) return TLC_ERR_INVALID_ARG;
    return run_accumulate_many(p, info->stream_bytes, payloads, in, in_stride, in_lens, scales, s, acc, workspace,
                               workspace_bytes, status, path_hint, dev_hint, static_cast<hipStream_t>(stream));
}

int tlc_copy_probe(const void* src, void* dst, uint64_t bytes, tlc_stream_t stream) {
    if (!src || !dst || (bytes & 15) || !aligned16(src) || !aligned16(dst)) return TLC_ERR_INVALID_ARG;
    if (bytes == 0) return TLC_OK;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const uint64_t n4 = bytes / 16;
    const uint64_t blocks = (n4 + kThreads - 1) / kThreads;
    if (blocks > 0xFFFFFFFFull) return TLC_ERR_INVALID_ARG;
    return launch("tlc_copy_probe", st, [&] {
        k_copy<<<(uint32_t)blocks, kThreads, 0, st>>>(static_cast<const float4*>(src), static_cast<float4*>(dst),
                                                       n4);
    });
}

int tlc_gather_probe(const float* src, const uint32_t* idx, uint64_t n, float* dst, tlc_stream_t stream) {
    if (!src || !idx || !dst || n == 0 || n > (1ull << 32)) return TLC_ERR_INVALID_ARG;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    return launch("tlc_gather_probe", st, [&] {
        k_gather<<<(uint32_t)((n + kThreads - 1) / kThreads), kThreads, 0, st>>>(src, idx, dst, n);
    });
}

int tlc_planes_gather(const float* src, const uint64_t* src_off, float* dst, const uint64_t* dst_off,
                      const uint64_t* n, uint32_t count, uint64_t max_n, tlc_stream_t stream) {
    return run_planes(true, src, src_off, dst, dst_off, n, count, max_n, static_cast<hipStream_t>(stream));
}

int tlc_planes_scatter(const float* src, const uint64_t* src_off, float* dst, const uint64_t* dst_off,
                       const uint64_t* n, uint32_t count, uint64_t max_n, tlc_stream_t stream) {
    return run_planes(false, src, src_off, dst, dst_off, n, count, max_n, static_cast<hipStream_t>(stream));
}

int tlc_profile_enable(int enable) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_on = enable != 0;
    return TLC_OK;
}

int tlc_profile_only(const char* kernel_name) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    memset(g_prof_only, 0, sizeof(g_prof_only));
    if (kernel_name) strncpy(g_prof_only, kernel_name, sizeof(g_prof_only) - 1);
    return TLC_OK;
}

int tlc_profile_read(tlc_kernel_time* out, int capacity, int* count) {
    std::vector<ProfRec> recs;
    {
        std::lock_guard<std::mutex> lk(g_prof_mu);
        recs.swap(g_prof);
    }
    int used = 0, rc = TLC_OK;
    for (const ProfRec& r : recs) {
        float ms = 0.0f;
        if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) rc = TLC_ERR_HIP;
        (void)hipEventDestroy(r.a);
        (void)hipEventDestroy(r.b);
        if (!out) continue;
        int k = 0;
        while (k < used && strcmp(out[k].name, r.name) != 0) ++k;
        if (k == used) {
            if (used == capacity) continue;
            memset(&out[k], 0, sizeof(out[k]));
            strncpy(out[k].name, r.name, sizeof(out[k].name) - 1);
            ++used;
        }
        out[k].launches += 1;
        out[k].total_ms += ms;
    }
    if (count) *count = used;
    return rc;
}

}  // extern "C"
