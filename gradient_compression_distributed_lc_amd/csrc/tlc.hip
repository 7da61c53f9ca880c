// tlc.hip -- 3LC state-change codec for AMD Instinct MI355X (gfx950).
//
// Implements the C ABI declared in include/tlc.h.  The codec is the one of
// the 3LC review page ("3LC: Lightweight and Effective Traffic Compression
// for Distributed Machine Learning", section "Proposed method"): error
// accumulation and 3-value quantization with a sparsity multiplier, quartic
// encoding (five ternary values per byte), zero-run encoding of the all-zero
// byte, and the reverse path.  The page's implementation is vectorised CPU
// code; here every step runs in the kernels below, laid out for CDNA4:
//
//   compress  = k_accum_max -> k_seg_scale -> k_encode
//     k_accum_max  one HBM pass over x and err: v = x + err written back to
//                  err, plus the max |v| of each 5120-element tile.  This is
//                  the 12-byte/element stream that bounds the codec.
//     k_seg_scale  one block per tensor: M = max of its tile maxima, M*s, and
//                  the fp32 selection threshold (see select_threshold).
//     k_encode     one block per tile, in ticket order.  A tile whose max is
//                  below the threshold holds only zero codes: it never touches
//                  x or err again and contributes a run of byte 121.  Other
//                  tiles re-read v, write err = v - q*M*s where q != 0, pack
//                  the quartic bytes in LDS and zero-run encode them.  The
//                  output position of every tile comes from a decoupled
//                  look-back scan whose carry is the small state (bytes
//                  emitted, pending run length mod 14).
//   decompress = k_fill_reset -> k_decode ; accumulate = k_reset -> k_decode
//     k_fill_reset dense zero fill of y (every code 0 dequantizes to +0.0)
//     k_decode     one block per 4096 stream bytes: expansion lengths, block
//                  scan, look-back scan for the quartic byte index, then only
//                  the literal bytes are decoded and their nonzero codes
//                  written (or added) to y.
//
// No matrix-core work exists on this path: it is bound by HBM bandwidth.

#include <hip/hip_runtime.h>

#include <float.h>
#include <limits.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "tlc.h"

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr uint32_t kTileElems = 5120;             // 1280 float4 = 5 per thread
constexpr uint32_t kTileBytes = kTileElems / 5;   // 1024 quartic bytes = 4 per thread
constexpr uint32_t kChunk = 4096;                 // decoder stream bytes per block = 16 per thread
constexpr uint32_t kZero = 121;                   // quartic byte of five zero codes
constexpr uint32_t kRunMax = 14;                  // codes 243..255 = runs of 2..14
constexpr uint32_t kRunBase = 241;
constexpr uint64_t kMaxN = 0xFFFFFFFFull;
constexpr uint32_t kSpinLimit = 1u << 20;         // bounded look-back wait (about a second)

// look-back word: 2 status bits | 62 payload bits
constexpr uint64_t kInvalid = 0, kAggregate = 1, kPrefix = 2, kPoison = 3;
constexpr uint64_t kPayloadMask = (1ull << 62) - 1;

struct Seg {
    uint64_t elem_off;    // first element in the flat fp32 buffers
    uint64_t n;           // elements
    uint64_t stream_off;  // first byte of this tensor's stream slot
    uint32_t tile0;       // first compress tile
    uint32_t chunk0;      // first decompress chunk
};
static_assert(sizeof(Seg) == 32, "table layout");

struct TableHeader {
    uint64_t magic, count, tiles, chunks, total_elems, stream_bytes, reserved0, reserved1;
};
static_assert(sizeof(TableHeader) == 64, "table layout");
constexpr uint64_t kMagic = 0x31434c5433ull;  // "3TLC1"

struct GroupView {
    const Seg* segs;          // device table, or nullptr for one tensor
    const uint32_t* tile_seg;
    const uint32_t* chunk_seg;
    Seg one;
};

__device__ __forceinline__ uint32_t tile_segment(const GroupView& g, uint32_t t) {
    return g.segs ? g.tile_seg[t] : 0u;
}
__device__ __forceinline__ uint32_t chunk_segment(const GroupView& g, uint32_t c) {
    return g.segs ? g.chunk_seg[c] : 0u;
}
__device__ __forceinline__ Seg load_seg(const GroupView& g, uint32_t i) {
    return g.segs ? g.segs[i] : g.one;
}

// ---------------------------------------------------------------------------
// wave / block primitives (wave64, 4 waves per block)

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

__device__ __forceinline__ float wave_max(float v) {
    for (int d = 32; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, 64));
    return v;
}

__device__ float block_max(float v, float* sm) {
    v = wave_max(v);
    if (lane_id() == 0) sm[wave_id()] = v;
    __syncthreads();
    float r = sm[0];
#pragma unroll
    for (int i = 1; i < kWaves; ++i) r = fmaxf(r, sm[i]);
    __syncthreads();
    return r;
}

__device__ int block_min_int(int v, int* sm) {
    for (int d = 32; d >= 1; d >>= 1) v = min(v, __shfl_xor(v, d, 64));
    if (lane_id() == 0) sm[wave_id()] = v;
    __syncthreads();
    int r = sm[0];
#pragma unroll
    for (int i = 1; i < kWaves; ++i) r = min(r, sm[i]);
    __syncthreads();
    return r;
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

// exclusive prefix max over the block (identity -1); *total receives the block max
__device__ int block_excl_max(int v, int* sm, int* total) {
    const int lane = lane_id(), w = wave_id();
    int inc = v;
    for (int d = 1; d < 64; d <<= 1) {
        int o = __shfl_up(inc, d, 64);
        if (lane >= d) inc = max(inc, o);
    }
    int prev = __shfl_up(inc, 1, 64);
    if (lane == 0) prev = -1;
    if (lane == 63) sm[w] = inc;
    __syncthreads();
    int before = -1, tot = -1;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        int t = sm[i];
        if (i < w) before = max(before, t);
        tot = max(tot, t);
    }
    __syncthreads();
    *total = tot;
    return max(before, prev);
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
// Payload bits: 61 = Lit, 60..57 = p, 56..53 = c, 31..0 = Q or K.

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

// ---------------------------------------------------------------------------
// compress kernels

__global__ __launch_bounds__(kThreads) void k_accum_max(GroupView g, const float* __restrict__ x,
                                                        float* __restrict__ err,
                                                        float* __restrict__ tile_max,
                                                        uint64_t* __restrict__ flags,
                                                        uint32_t* __restrict__ ctrl,
                                                        int* __restrict__ status) {
    __shared__ float sm[kWaves];
    const uint32_t tile = blockIdx.x;
    const Seg sg = load_seg(g, tile_segment(g, tile));
    const uint64_t lt = tile - sg.tile0;
    const uint64_t e0 = sg.elem_off + lt * kTileElems;
    const uint64_t e1 = min(sg.elem_off + sg.n, e0 + kTileElems);
    float m = 0.0f;
    if ((e0 & 3) == 0 && e1 - e0 == kTileElems) {
        const float4* xs = reinterpret_cast<const float4*>(x + e0);
        float4* es = reinterpret_cast<float4*>(err + e0);
        float4 a[5], b[5];
#pragma unroll
        for (int k = 0; k < 5; ++k) {
            a[k] = xs[threadIdx.x + k * kThreads];
            b[k] = es[threadIdx.x + k * kThreads];
        }
#pragma unroll
        for (int k = 0; k < 5; ++k) {
            const float4 v = make_float4(a[k].x + b[k].x, a[k].y + b[k].y, a[k].z + b[k].z, a[k].w + b[k].w);
            es[threadIdx.x + k * kThreads] = v;
            m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
        }
    } else {
        for (uint64_t i = e0 + threadIdx.x; i < e1; i += kThreads) {
            const float v = x[i] + err[i];
            err[i] = v;
            m = fmaxf(m, fabsf(v));
        }
    }
    m = block_max(m, sm);
    if (threadIdx.x == 0) {
        tile_max[tile] = m;
        flags[tile] = 0;
        if (tile == 0) {
            ctrl[0] = 0;
            *status = TLC_OK;
        }
    }
}

__global__ __launch_bounds__(kThreads) void k_seg_scale(GroupView g, float s, const float* __restrict__ tile_max,
                                                        float* __restrict__ scales, float* __restrict__ seg_thr,
                                                        float* __restrict__ seg_ms) {
    __shared__ float sm[kWaves];
    const uint32_t si = blockIdx.x;
    const Seg sg = load_seg(g, si);
    const uint32_t nt = (uint32_t)((sg.n + kTileElems - 1) / kTileElems);
    float m = 0.0f;
    for (uint32_t t = threadIdx.x; t < nt; t += kThreads) m = fmaxf(m, tile_max[sg.tile0 + t]);
    m = block_max(m, sm);
    if (threadIdx.x == 0) {
        const float ms = m * s;
        scales[si] = m;
        seg_ms[si] = ms;
        seg_thr[si] = select_threshold(m, ms);
    }
}

__global__ __launch_bounds__(kThreads) void k_encode(GroupView g, float* __restrict__ err,
                                                     const float* __restrict__ tile_max,
                                                     const float* __restrict__ seg_thr,
                                                     const float* __restrict__ seg_ms,
                                                     uint64_t* __restrict__ flags, uint32_t* __restrict__ ctrl,
                                                     uint8_t* __restrict__ out, uint64_t* __restrict__ out_lens,
                                                     int* __restrict__ status) {
    __shared__ __align__(16) int8_t s_q[kTileElems];
    __shared__ uint32_t s_u[kWaves];
    __shared__ int s_i[kWaves];
    __shared__ uint32_t s_tile, s_E, s_r, s_ok;

    if (threadIdx.x == 0) s_tile = atomicAdd(ctrl, 1u);
    __syncthreads();
    const uint32_t tile = s_tile;
    const uint32_t si = tile_segment(g, tile);
    const Seg sg = load_seg(g, si);
    const uint32_t lt = tile - sg.tile0;
    const uint32_t n = (uint32_t)sg.n;
    const uint32_t B = (uint32_t)(((uint64_t)n + 4) / 5);
    const uint32_t nt = (uint32_t)(((uint64_t)n + kTileElems - 1) / kTileElems);
    const uint32_t nbytes = min(kTileBytes, B - lt * kTileBytes);
    const uint32_t nel = min(kTileElems, n - lt * kTileElems);
    const uint64_t e0 = sg.elem_off + (uint64_t)lt * kTileElems;
    const float thr = seg_thr[si];
    const float ms = seg_ms[si];
    const bool active = tile_max[tile] >= thr;  // same for every thread
    uint8_t* const o = out + sg.stream_off;

    Carry agg = carry_run(nbytes);
    uint32_t b[4] = {kZero, kZero, kZero, kZero};
    const uint32_t kb = 4 * threadIdx.x;  // this thread's first tile byte
    int first = INT_MAX, last = -1, prev_excl = -1;
    uint32_t emit_excl = 0, k_int = 0;

    if (active) {
        // ternary codes of the tile into LDS; pad codes past the tensor are 0
        for (uint32_t u = nel + threadIdx.x; u < 5 * nbytes; u += kThreads) s_q[u] = 0;
        if ((e0 & 3) == 0 && nel == kTileElems) {
            float4* es = reinterpret_cast<float4*>(err + e0);
            float4 v[5];
#pragma unroll
            for (int k = 0; k < 5; ++k) v[k] = es[threadIdx.x + k * kThreads];
#pragma unroll
            for (int k = 0; k < 5; ++k) {
                const uint32_t slot = threadIdx.x + k * kThreads;
                const float vv[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
                uint32_t packed = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int q = fabsf(vv[j]) >= thr ? (vv[j] > 0.0f ? 1 : -1) : 0;
                    if (q) err[e0 + 4 * slot + j] = vv[j] - (float)q * ms;
                    packed |= (uint32_t)(uint8_t)(int8_t)q << (8 * j);
                }
                reinterpret_cast<uint32_t*>(s_q)[slot] = packed;
            }
        } else {
            for (uint32_t u = threadIdx.x; u < nel; u += kThreads) {
                const float vv = err[e0 + u];
                const int q = fabsf(vv) >= thr ? (vv > 0.0f ? 1 : -1) : 0;
                if (q) err[e0 + u] = vv - (float)q * ms;
                s_q[u] = (int8_t)q;
            }
        }
        __syncthreads();

        // quartic bytes 4t..4t+3 from codes 20t..20t+19
        uint32_t words[5];
#pragma unroll
        for (int i = 0; i < 5; ++i) words[i] = reinterpret_cast<const uint32_t*>(s_q)[5 * threadIdx.x + i];
        int tfirst = INT_MAX, tlast = -1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t byte = 0, w3 = 1;
#pragma unroll
            for (int d = 0; d < 5; ++d) {
                const int idx = 5 * j + d;
                const int q = (int)(int8_t)(words[idx >> 2] >> (8 * (idx & 3)));
                byte += (uint32_t)(q + 1) * w3;
                w3 *= 3;
            }
            const uint32_t k = kb + j;
            if (k < nbytes) {
                b[j] = byte;
                if (byte != kZero) {
                    tfirst = min(tfirst, (int)k);
                    tlast = (int)k;
                }
            }
        }
        prev_excl = block_excl_max(tlast, s_i, &last);
        first = block_min_int(tfirst, s_i);

        if (last >= 0) {
            // stream bytes emitted from the first literal on: a literal emits
            // the remainder code of the run before it (if any) and itself; a
            // 121 emits a 255 when it completes a 14-byte chunk of its run
            uint32_t te = 0;
            int prev = prev_excl;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int k = (int)kb + j;
                if (k < (int)nbytes && k >= first) {
                    if (b[j] != kZero) {
                        te += (k == first) ? 1u : 1u + (((k - prev - 1) % (int)kRunMax) != 0);
                        prev = k;
                    } else {
                        te += ((k - prev) % (int)kRunMax) == 0;
                    }
                }
            }
            emit_excl = block_excl_sum(te, s_u, &k_int);
            agg.lit = 1;
            agg.p = (uint32_t)first % kRunMax;
            agg.K = (uint32_t)first / kRunMax + k_int;
            agg.c = (nbytes - 1 - (uint32_t)last) % kRunMax;
        }
    }

    // publish this tile's summary, look back for the state before it
    if (threadIdx.x < 64) {
        uint32_t E = 0, r = 0, ok = 1;
        if (lt == 0) {
            if (threadIdx.x == 0) {
                uint32_t E2, r2;
                carry_apply(agg, 0, 0, &E2, &r2);
                publish(flags, tile, kPrefix, (uint64_t)E2 | ((uint64_t)r2 << 57));
            }
        } else {
            if (threadIdx.x == 0) publish(flags, tile, kAggregate, carry_pack(agg));
            uint64_t f = 0;
            ok = look_back(flags, tile, sg.tile0, carry_pack(carry_run(0)), CarryCompose(), &f) ? 1u : 0u;
            if (ok) carry_apply(carry_unpack(f), 0, 0, &E, &r);
            if (threadIdx.x == 0) {
                if (ok) {
                    uint32_t E2, r2;
                    carry_apply(agg, E, r, &E2, &r2);
                    publish(flags, tile, kPrefix, (uint64_t)E2 | ((uint64_t)r2 << 57));
                } else {
                    publish(flags, tile, kPoison, 0);
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
    const uint32_t E_in = s_E, r_in = s_r;
    uint32_t E_out, r_out;
    if (!agg.lit) {
        const uint32_t t = r_in + nbytes;
        const uint32_t n255 = t / kRunMax;
        for (uint32_t i = threadIdx.x; i < n255; i += kThreads)
            if (E_in + i < B) o[E_in + i] = 255;
        E_out = E_in + n255;
        r_out = t % kRunMax;
    } else {
        const uint32_t t = r_in + (uint32_t)first;
        const uint32_t n255 = t / kRunMax, rem = t % kRunMax;
        for (uint32_t i = threadIdx.x; i < n255; i += kThreads)
            if (E_in + i < B) o[E_in + i] = 255;
        if (rem && threadIdx.x == 0 && E_in + n255 < B) o[E_in + n255] = remainder_code(rem);
        const uint32_t base = E_in + n255 + (rem ? 1u : 0u);
        uint32_t pos = base + emit_excl;
        int prev = prev_excl;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int k = (int)kb + j;
            if (k < (int)nbytes && k >= first) {
                if (b[j] != kZero) {
                    if (k != first) {
                        const uint32_t gap = (uint32_t)((k - prev - 1) % (int)kRunMax);
                        if (gap) {
                            if (pos < B) o[pos] = remainder_code(gap);
                            ++pos;
                        }
                    }
                    if (pos < B) o[pos] = (uint8_t)b[j];
                    ++pos;
                    prev = k;
                } else if (((k - prev) % (int)kRunMax) == 0) {
                    if (pos < B) o[pos] = 255;
                    ++pos;
                }
            }
        }
        E_out = base + k_int;
        r_out = agg.c;
    }
    if (lt == nt - 1 && threadIdx.x == 0) {
        // the stream never outgrows ceil(n/5); the guards above keep even a
        // wrong length from writing past the tensor's slot
        const uint64_t len = (uint64_t)E_out + (r_out ? 1u : 0u);
        if (r_out && E_out < B) o[E_out] = remainder_code(r_out);
        if (len > B) raise_status(status, TLC_ERR_INTERNAL);
        out_lens[si] = len;
    }
}

// ---------------------------------------------------------------------------
// decompress kernels

__global__ __launch_bounds__(kThreads) void k_fill_reset(float* __restrict__ y, uint64_t n,
                                                         uint64_t* __restrict__ flags, uint64_t nflags,
                                                         uint32_t* __restrict__ ctrl, int* __restrict__ status) {
    const uint64_t n4 = n >> 2;
    const uint64_t stride = (uint64_t)gridDim.x * kThreads;
    const uint64_t tid = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
    float4* y4 = reinterpret_cast<float4*>(y);
    const float4 z = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (uint64_t i = tid; i < n4; i += stride) y4[i] = z;
    if (tid < (n & 3)) y[(n4 << 2) + tid] = 0.0f;
    for (uint64_t i = tid; i < nflags; i += stride) flags[i] = 0;
    if (tid == 0) {
        ctrl[1] = 0;
        *status = TLC_OK;
    }
}

__global__ __launch_bounds__(kThreads) void k_reset(uint64_t* __restrict__ flags, uint64_t nflags,
                                                    uint32_t* __restrict__ ctrl, int* __restrict__ status) {
    const uint64_t stride = (uint64_t)gridDim.x * kThreads;
    const uint64_t tid = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
    for (uint64_t i = tid; i < nflags; i += stride) flags[i] = 0;
    if (tid == 0) {
        ctrl[1] = 0;
        *status = TLC_OK;
    }
}

__global__ __launch_bounds__(kThreads) void k_decode(GroupView g, const uint8_t* __restrict__ in,
                                                     const uint64_t* __restrict__ in_lens,
                                                     const float* __restrict__ scales, float s,
                                                     float* __restrict__ y, uint64_t* __restrict__ flags,
                                                     uint32_t* __restrict__ ctrl, int* __restrict__ status,
                                                     int accumulate) {
    __shared__ uint32_t s_u[kWaves];
    __shared__ uint32_t s_chunk, s_ok;
    __shared__ uint64_t s_base;

    if (threadIdx.x == 0) s_chunk = atomicAdd(ctrl + 1, 1u);
    __syncthreads();
    const uint32_t c = s_chunk;
    const uint32_t si = chunk_segment(g, c);
    const Seg sg = load_seg(g, si);
    const uint32_t lc = c - sg.chunk0;
    const uint32_t n = (uint32_t)sg.n;
    const uint64_t B = ((uint64_t)n + 4u) / 5u;
    uint64_t L = in_lens[si];
    if (L > B) {
        if (lc == 0 && threadIdx.x == 0) raise_status(status, TLC_ERR_CORRUPT);
        L = B;
    }
    const uint64_t start = (uint64_t)lc * kChunk;
    if (start >= L) {
        // past the end of this stream (or an empty stream, which is corrupt
        // because ceil(n/5) >= 1); later chunks of the tensor exit here too,
        // so nothing waits for this block
        if (lc == 0 && threadIdx.x == 0) raise_status(status, TLC_ERR_CORRUPT);
        return;
    }
    const uint32_t cnt = (uint32_t)min((uint64_t)kChunk, L - start);
    const uint8_t* p = in + sg.stream_off + start;
    const uint32_t off = 16u * threadIdx.x;
    const uint32_t nv = cnt > off ? min(16u, cnt - off) : 0u;
    uint32_t w[4] = {0, 0, 0, 0};
    if (nv == 16 && ((reinterpret_cast<uintptr_t>(p + off) & 15) == 0)) {
        const uint4 v = *reinterpret_cast<const uint4*>(p + off);
        w[0] = v.x;
        w[1] = v.y;
        w[2] = v.z;
        w[3] = v.w;
    } else {
        for (uint32_t i = 0; i < nv; ++i) w[i >> 2] |= (uint32_t)p[off + i] << (8 * (i & 3));
    }
    uint32_t tsum = 0;
#pragma unroll
    for (uint32_t i = 0; i < 16; ++i) {
        const uint32_t byte = (w[i >> 2] >> (8 * (i & 3))) & 255u;
        tsum += (i < nv) ? (byte < 243u ? 1u : byte - kRunBase) : 0u;
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
            ok = look_back(flags, c, sg.chunk0, 0, SumCompose(), &base) ? 1u : 0u;
            if (threadIdx.x == 0) publish(flags, c, ok ? kPrefix : kPoison, base + csum);
        }
        if (threadIdx.x == 0) {
            s_base = base;
            s_ok = ok;
        }
    }
    __syncthreads();
    if (!s_ok) {
        if (threadIdx.x == 0) raise_status(status, TLC_ERR_INTERNAL);
        return;
    }
    const uint64_t base = s_base;
    const float ms = scales[si] * s;
    float* const yy = y + sg.elem_off;
    uint64_t pos = base + texcl;
    bool bad = false;
    for (uint32_t i = 0; i < nv; ++i) {
        const uint32_t byte = (w[i >> 2] >> (8 * (i & 3))) & 255u;
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
                        yy[e] = accumulate ? yy[e] + val : val;
                    }
                }
            }
            pos += 1;
        } else {
            pos += byte - kRunBase;
        }
    }
    if (bad) raise_status(status, TLC_ERR_CORRUPT);
    if (threadIdx.x == 0 && start + cnt == L && base + csum != B) raise_status(status, TLC_ERR_CORRUPT);
}

// ---------------------------------------------------------------------------
// bandwidth yardstick

__global__ __launch_bounds__(kThreads) void k_copy(const float4* __restrict__ src, float4* __restrict__ dst,
                                                   uint64_t n4) {
    const uint64_t stride = (uint64_t)gridDim.x * kThreads;
    for (uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x; i < n4; i += stride) dst[i] = src[i];
}

// ---------------------------------------------------------------------------
// host side

struct ProfRec {
    const char* name;
    hipEvent_t a, b;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRec> g_prof;

template <typename Launch>
int launch(const char* name, hipStream_t st, Launch&& fn) {
    hipEvent_t a = nullptr, b = nullptr;
    bool prof;
    {
        std::lock_guard<std::mutex> lk(g_prof_mu);
        prof = g_prof_on;
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

constexpr size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

struct Layout {
    size_t ctrl, tile_max, enc_flags, seg_thr, seg_ms, dec_flags, total;
};

Layout ws_layout(uint64_t count, uint64_t tiles, uint64_t chunks) {
    Layout l;
    size_t off = 0;
    l.ctrl = off;
    off += 256;
    l.tile_max = off;
    off = align_up(off + tiles * sizeof(float), 256);
    l.enc_flags = off;
    off = align_up(off + tiles * sizeof(uint64_t), 256);
    l.seg_thr = off;
    off = align_up(off + count * sizeof(float), 256);
    l.seg_ms = off;
    off = align_up(off + count * sizeof(float), 256);
    l.dec_flags = off;
    off = align_up(off + chunks * sizeof(uint64_t), 256);
    l.total = off;
    return l;
}

uint64_t tiles_of(uint64_t n) { return (n + kTileElems - 1) / kTileElems; }
uint64_t chunks_of(uint64_t n) { return ((n + 4) / 5 + kChunk - 1) / kChunk; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
bool valid_s(float s) { return s >= 1.0f && s < 2.0f; }  // false for NaN

struct Plan {
    GroupView g;
    uint64_t count, tiles, chunks, total_elems;
};

Plan single_plan(uint64_t n) {
    Plan p;
    p.g.segs = nullptr;
    p.g.tile_seg = nullptr;
    p.g.chunk_seg = nullptr;
    p.g.one.elem_off = 0;
    p.g.one.n = n;
    p.g.one.stream_off = 0;
    p.g.one.tile0 = 0;
    p.g.one.chunk0 = 0;
    p.count = 1;
    p.tiles = tiles_of(n);
    p.chunks = chunks_of(n);
    p.total_elems = n;
    return p;
}

struct TableLayout {
    size_t segs, tile_seg, chunk_seg, total;
};
TableLayout table_layout(uint64_t count, uint64_t tiles, uint64_t chunks) {
    TableLayout t;
    t.segs = sizeof(TableHeader);
    t.tile_seg = align_up(t.segs + count * sizeof(Seg), 16);
    t.chunk_seg = align_up(t.tile_seg + tiles * sizeof(uint32_t), 16);
    t.total = align_up(t.chunk_seg + chunks * sizeof(uint32_t), 16);
    return t;
}

int group_plan_of(const tlc_group_info* info, const void* d_table, Plan* p) {
    if (!info || !d_table || !aligned16(d_table) || info->count == 0) return TLC_ERR_INVALID_ARG;
    const TableLayout t = table_layout(info->count, info->tiles, info->chunks);
    if (t.total != info->table_bytes) return TLC_ERR_INVALID_ARG;
    const char* base = static_cast<const char*>(d_table);
    p->g.segs = reinterpret_cast<const Seg*>(base + t.segs);
    p->g.tile_seg = reinterpret_cast<const uint32_t*>(base + t.tile_seg);
    p->g.chunk_seg = reinterpret_cast<const uint32_t*>(base + t.chunk_seg);
    memset(&p->g.one, 0, sizeof(Seg));
    p->count = info->count;
    p->tiles = info->tiles;
    p->chunks = info->chunks;
    p->total_elems = info->total_elems;
    return TLC_OK;
}

int check_ws(const Plan& p, void* ws, size_t ws_bytes, Layout* l) {
    *l = ws_layout(p.count, p.tiles, p.chunks);
    if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255) || ws_bytes < l->total) return TLC_ERR_WORKSPACE;
    return TLC_OK;
}

int run_compress(const Plan& p, const float* x, float* err, float s, uint8_t* out, uint64_t* out_lens,
                 float* scales, void* ws, size_t ws_bytes, int* status, hipStream_t st) {
    if (!x || !err || !out || !out_lens || !scales || !status) return TLC_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(err) || !valid_s(s)) return TLC_ERR_INVALID_ARG;
    Layout l;
    int rc = check_ws(p, ws, ws_bytes, &l);
    if (rc) return rc;
    char* w = static_cast<char*>(ws);
    uint32_t* ctrl = reinterpret_cast<uint32_t*>(w + l.ctrl);
    float* tile_max = reinterpret_cast<float*>(w + l.tile_max);
    uint64_t* flags = reinterpret_cast<uint64_t*>(w + l.enc_flags);
    float* thr = reinterpret_cast<float*>(w + l.seg_thr);
    float* ms = reinterpret_cast<float*>(w + l.seg_ms);
    const GroupView g = p.g;
    const uint32_t tiles = (uint32_t)p.tiles, count = (uint32_t)p.count;
    rc = launch("tlc_accum_max", st, [&] {
        k_accum_max<<<tiles, kThreads, 0, st>>>(g, x, err, tile_max, flags, ctrl, status);
    });
    if (rc) return rc;
    rc = launch("tlc_seg_scale", st, [&] {
        k_seg_scale<<<count, kThreads, 0, st>>>(g, s, tile_max, scales, thr, ms);
    });
    if (rc) return rc;
    return launch("tlc_encode", st, [&] {
        k_encode<<<tiles, kThreads, 0, st>>>(g, err, tile_max, thr, ms, flags, ctrl, out, out_lens, status);
    });
}

int run_decompress(const Plan& p, const uint8_t* in, const uint64_t* in_lens, const float* scales, float s,
                   float* y, void* ws, size_t ws_bytes, int* status, hipStream_t st, int accumulate) {
    if (!in || !in_lens || !scales || !y || !status) return TLC_ERR_INVALID_ARG;
    if (!aligned16(y) || !valid_s(s)) return TLC_ERR_INVALID_ARG;
    Layout l;
    int rc = check_ws(p, ws, ws_bytes, &l);
    if (rc) return rc;
    char* w = static_cast<char*>(ws);
    uint32_t* ctrl = reinterpret_cast<uint32_t*>(w + l.ctrl);
    uint64_t* flags = reinterpret_cast<uint64_t*>(w + l.dec_flags);
    const GroupView g = p.g;
    const uint64_t chunks = p.chunks;
    if (accumulate) {
        const uint32_t grid = (uint32_t)std::min<uint64_t>(1024, (chunks + kThreads - 1) / kThreads + 1);
        rc = launch("tlc_reset", st, [&] { k_reset<<<grid, kThreads, 0, st>>>(flags, chunks, ctrl, status); });
    } else {
        const uint64_t n4 = p.total_elems >> 2;
        uint64_t blocks = (n4 + kThreads * 8 - 1) / (kThreads * 8);
        blocks = std::max<uint64_t>(blocks, (chunks + kThreads - 1) / kThreads);
        blocks = std::max<uint64_t>(blocks, 1);
        const uint32_t grid = (uint32_t)std::min<uint64_t>(blocks, 1u << 20);
        rc = launch("tlc_fill_reset", st, [&] {
            k_fill_reset<<<grid, kThreads, 0, st>>>(y, p.total_elems, flags, chunks, ctrl, status);
        });
    }
    if (rc) return rc;
    return launch("tlc_decode", st, [&] {
        k_decode<<<(uint32_t)chunks, kThreads, 0, st>>>(g, in, in_lens, scales, s, y, flags, ctrl, status,
                                                         accumulate);
    });
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI

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
        default: return "unknown status";
    }
}

const char* tlc_version(void) { return "tlc-gfx950 0.1"; }

uint64_t tlc_compress_bound(uint64_t n) { return (n + 4) / 5; }

size_t tlc_workspace_size(uint64_t n) {
    if (n == 0 || n > kMaxN) return 0;
    return ws_layout(1, tiles_of(n), chunks_of(n)).total;
}

int tlc_compress(const float* x, float* err, uint64_t n, float s, uint8_t* out, uint64_t out_capacity,
                 uint64_t* out_len, float* scale, void* workspace, size_t workspace_bytes, int* status,
                 tlc_stream_t stream) {
    if (n == 0 || n > kMaxN) return TLC_ERR_INVALID_ARG;
    if (out_capacity < tlc_compress_bound(n)) return TLC_ERR_CAPACITY;
    return run_compress(single_plan(n), x, err, s, out, out_len, scale, workspace, workspace_bytes, status,
                        static_cast<hipStream_t>(stream));
}

int tlc_decompress(const uint8_t* in, const uint64_t* in_len, const float* scale, uint64_t n, float s, float* y,
                   void* workspace, size_t workspace_bytes, int* status, tlc_stream_t stream) {
    if (n == 0 || n > kMaxN) return TLC_ERR_INVALID_ARG;
    return run_decompress(single_plan(n), in, in_len, scale, s, y, workspace, workspace_bytes, status,
                          static_cast<hipStream_t>(stream), 0);
}

int tlc_decompress_accumulate(const uint8_t* in, const uint64_t* in_len, const float* scale, uint64_t n, float s,
                              float* acc, void* workspace, size_t workspace_bytes, int* status,
                              tlc_stream_t stream) {
    if (n == 0 || n > kMaxN) return TLC_ERR_INVALID_ARG;
    return run_decompress(single_plan(n), in, in_len, scale, s, acc, workspace, workspace_bytes, status,
                          static_cast<hipStream_t>(stream), 1);
}

int tlc_group_plan(const uint64_t* sizes, uint64_t count, tlc_group_info* info, void* table,
                   size_t table_capacity, uint64_t* stream_offset) {
    if (!sizes || !info || count == 0 || count > 0xFFFFFFFFull) return TLC_ERR_INVALID_ARG;
    uint64_t tiles = 0, chunks = 0, elems = 0, stream = 0;
    for (uint64_t i = 0; i < count; ++i) {
        const uint64_t n = sizes[i];
        if (n == 0 || n > kMaxN) return TLC_ERR_INVALID_ARG;
        tiles += tiles_of(n);
        chunks += chunks_of(n);
        elems += n;
        stream = align_up(stream, 16) + tlc_compress_bound(n);
    }
    if (tiles > 0xFFFFFFFFull || chunks > 0xFFFFFFFFull) return TLC_ERR_INVALID_ARG;
    const TableLayout t = table_layout(count, tiles, chunks);
    info->count = count;
    info->total_elems = elems;
    info->stream_bytes = align_up(stream, 16);
    info->table_bytes = t.total;
    info->workspace_bytes = ws_layout(count, tiles, chunks).total;
    info->tiles = tiles;
    info->chunks = chunks;
    if (!table && !stream_offset) return TLC_OK;
    if (table && table_capacity < t.total) return TLC_ERR_CAPACITY;
    char* base = static_cast<char*>(table);
    if (table) {
        memset(base, 0, t.total);
        TableHeader h = {kMagic, count, tiles, chunks, elems, info->stream_bytes, 0, 0};
        memcpy(base, &h, sizeof(h));
    }
    uint64_t tile = 0, chunk = 0, eoff = 0, soff = 0;
    for (uint64_t i = 0; i < count; ++i) {
        const uint64_t n = sizes[i];
        soff = align_up(soff, 16);
        if (stream_offset) stream_offset[i] = soff;
        if (table) {
            Seg sg;
            sg.elem_off = eoff;
            sg.n = n;
            sg.stream_off = soff;
            sg.tile0 = (uint32_t)tile;
            sg.chunk0 = (uint32_t)chunk;
            memcpy(base + t.segs + i * sizeof(Seg), &sg, sizeof(Seg));
            uint32_t* ts = reinterpret_cast<uint32_t*>(base + t.tile_seg);
            uint32_t* cs = reinterpret_cast<uint32_t*>(base + t.chunk_seg);
            for (uint64_t k = 0; k < tiles_of(n); ++k) ts[tile + k] = (uint32_t)i;
            for (uint64_t k = 0; k < chunks_of(n); ++k) cs[chunk + k] = (uint32_t)i;
        }
        tile += tiles_of(n);
        chunk += chunks_of(n);
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
    return run_compress(p, x, err, s, out, out_lens, scales, workspace, workspace_bytes, status,
                        static_cast<hipStream_t>(stream));
}

int tlc_decompress_group(const tlc_group_info* info, const void* d_table, const uint8_t* in,
                         const uint64_t* in_lens, const float* scales, float s, float* y, void* workspace,
                         size_t workspace_bytes, int* status, tlc_stream_t stream) {
    Plan p;
    int rc = group_plan_of(info, d_table, &p);
    if (rc) return rc;
    return run_decompress(p, in, in_lens, scales, s, y, workspace, workspace_bytes, status,
                          static_cast<hipStream_t>(stream), 0);
}

int tlc_decompress_accumulate_group(const tlc_group_info* info, const void* d_table, const uint8_t* in,
                                    const uint64_t* in_lens, const float* scales, float s, float* acc,
                                    void* workspace, size_t workspace_bytes, int* status, tlc_stream_t stream) {
    Plan p;
    int rc = group_plan_of(info, d_table, &p);
    if (rc) return rc;
    return run_decompress(p, in, in_lens, scales, s, acc, workspace, workspace_bytes, status,
                          static_cast<hipStream_t>(stream), 1);
}

int tlc_copy_probe(const void* src, void* dst, uint64_t bytes, tlc_stream_t stream) {
    if (!src || !dst || (bytes & 15) || !aligned16(src) || !aligned16(dst)) return TLC_ERR_INVALID_ARG;
    if (bytes == 0) return TLC_OK;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const uint64_t n4 = bytes / 16;
    const uint32_t grid = (uint32_t)std::min<uint64_t>((n4 + kThreads * 8 - 1) / (kThreads * 8), 1u << 20);
    return launch("tlc_copy_probe", st, [&] {
        k_copy<<<grid, kThreads, 0, st>>>(static_cast<const float4*>(src), static_cast<float4*>(dst), n4);
    });
}

int tlc_profile_enable(int enable) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_on = enable != 0;
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
