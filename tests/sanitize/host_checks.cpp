// Host-only checks of libtlc, built together with tlc.hip with
// AddressSanitizer and UndefinedBehaviorSanitizer on the host code: the group
// planner over ragged groups (sizes 1 to 2^32-1, thousands of tensors), the
// workspace and table sizes it reports, the table and stream offsets it
// writes (bounds and alignment, against sizes derived here from the
// documented layout), its refusals, and the argument checks every entry
// point makes before any launch.  Nothing here touches a GPU: device
// pointers are fake addresses that every call rejects before using them.
#include <algorithm>
#include <cinttypes>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "tlc.h"

static int failures = 0;
#define CHECK(cond)                                                          \
    do {                                                                     \
        if (!(cond)) {                                                       \
            std::fprintf(stderr, "check failed, line %d: %s\n", __LINE__, #cond); \
            ++failures;                                                      \
        }                                                                    \
    } while (0)

static uint64_t ceil_div(uint64_t a, uint64_t b) { return (a + b - 1) / b; }

// Plan a group and check what the planner reports against the layout the
// header documents.
static void check_plan(const std::vector<uint64_t>& sizes) {
    tlc_group_info info{};
    CHECK(tlc_group_plan(sizes.data(), sizes.size(), &info, nullptr, 0, nullptr) == TLC_OK);
    uint64_t total = 0, tiles = 0, chunks = 0, spans = 0, stream = 0;
    for (uint64_t n : sizes) {
        total += n;
        tiles += ceil_div(n, 5120);
        spans += ceil_div(ceil_div(n, 5120), 256);
        chunks += std::max<uint64_t>(1, ceil_div(ceil_div(n, 5), 4096));
        stream = (stream + 15) / 16 * 16 + ceil_div(n, 5);
    }
    CHECK(info.count == sizes.size());
    CHECK(info.total_elems == total);
    CHECK(info.tiles == tiles && info.spans == spans && info.chunks == chunks);
    CHECK(info.stream_bytes == (stream + 15) / 16 * 16);
    CHECK(info.table_bytes > 0 && info.table_bytes % 16 == 0);
    CHECK(info.workspace_bytes > 0 && info.workspace_bytes % 256 == 0);
    // the table and the offsets, written into exactly sized buffers (ASan
    // reports any write past them)
    std::vector<unsigned char> table(info.table_bytes);
    std::vector<uint64_t> offs(sizes.size());
    tlc_group_info again{};
    CHECK(tlc_group_plan(sizes.data(), sizes.size(), &again, table.data(), table.size(), offs.data()) == TLC_OK);
    CHECK(again.table_bytes == info.table_bytes && again.workspace_bytes == info.workspace_bytes);
    uint64_t end = 0;
    for (size_t t = 0; t < sizes.size(); ++t) {
        CHECK(offs[t] % 16 == 0 && offs[t] >= end);
        end = offs[t] + ceil_div(sizes[t], 5);
    }
    CHECK(end <= info.stream_bytes);
    // one byte short of the table: refused, nothing written past it
    if (info.table_bytes > 16) {
        std::vector<unsigned char> small(info.table_bytes - 1);
        CHECK(tlc_group_plan(sizes.data(), sizes.size(), &again, small.data(), small.size(), nullptr) ==
              TLC_ERR_CAPACITY);
    }
    // workspace of the many-payload accumulate: grows with the payloads,
    // refused outside 1..64
    uint64_t prev = 0;
    for (uint32_t P = 1; P <= 64; P *= 2) {
        const uint64_t w = tlc_accumulate_many_workspace_size(&info, P);
        CHECK(w > 0 && w % 256 == 0 && w >= prev);
        prev = w;
    }
    CHECK(tlc_accumulate_many_workspace_size(&info, 0) == 0);
    CHECK(tlc_accumulate_many_workspace_size(&info, 65) == 0);
    CHECK(tlc_accumulate_many_workspace_size(nullptr, 1) == 0);
    // the wire message: 8 header bytes per tensor plus every slot, and a
    // workspace of the stream offsets, chunk numbers and one control block
    CHECK(tlc_wire_bound(&info) == 8 * info.count + info.stream_bytes);
    const uint64_t ww = tlc_wire_workspace_size(&info);
    CHECK(ww % 256 == 0 && ww >= 8 * (info.count + 1) + 4 * info.count + 256);
}

int main() {
    std::mt19937_64 rng(2024);
    // ragged groups: log-uniform sizes, boundary sizes around tiles, chunks and spans
    const uint64_t edges[] = {1, 4, 5, 6, 511, 512, 513, 5119, 5120, 5121, 20479, 20480, 20481,
                              5120ull * 256 - 1, 5120ull * 256, 5120ull * 256 + 1};
    for (int trial = 0; trial < 60; ++trial) {
        std::vector<uint64_t> sizes(1 + rng() % (trial < 30 ? 40 : 3000));
        for (auto& n : sizes) {
            const uint32_t r = (uint32_t)(rng() % 10);
            if (r < 2)
                n = edges[rng() % (sizeof(edges) / sizeof(edges[0]))];
            else
                n = 1 + (uint64_t)std::exp(std::uniform_real_distribution<double>(0.0, std::log(1 << 22))(rng));
        }
        check_plan(sizes);
    }
    // the largest tensors
    check_plan({4294967295ull});
    check_plan({4294967295ull, 1, 4294967295ull, 7});
    // refusals
    tlc_group_info info{};
    const uint64_t too_big[] = {4294967296ull}, zero[] = {5, 0}, ok[] = {100};
    CHECK(tlc_group_plan(too_big, 1, &info, nullptr, 0, nullptr) == TLC_ERR_INVALID_ARG);
    CHECK(tlc_group_plan(zero, 2, &info, nullptr, 0, nullptr) == TLC_ERR_INVALID_ARG);
    CHECK(tlc_group_plan(ok, 0, &info, nullptr, 0, nullptr) == TLC_ERR_INVALID_ARG);
    CHECK(tlc_group_plan(nullptr, 1, &info, nullptr, 0, nullptr) == TLC_ERR_INVALID_ARG);
    CHECK(tlc_group_plan(ok, 1, nullptr, nullptr, 0, nullptr) == TLC_ERR_INVALID_ARG);

    // bounds and sizes of the single-tensor calls
    CHECK(tlc_compress_bound(1) == 1 && tlc_compress_bound(4294967295ull) == 858993459ull);
    CHECK(tlc_workspace_size(0) == 0 && tlc_workspace_size(4294967296ull) == 0);
    CHECK(tlc_workspace_size(1) > 0 && tlc_workspace_size(4294967295ull) > tlc_workspace_size(1));
    CHECK(tlc_fixed_len(10, TLC_ENC_TWOBIT) == 3 && tlc_fixed_len(10, 9) == 0);
    CHECK(tlc_compress_static_max_n() > 0);
    for (int code = -1; code < 12; ++code) CHECK(tlc_status_string(code) != nullptr);

    // argument checks before any launch; fake device addresses are never used
    void* const fake = reinterpret_cast<void*>(0x10000);
    void* const odd = reinterpret_cast<void*>(0x10004);
    void* const ws = reinterpret_cast<void*>(0x20000);
    float* const ff = static_cast<float*>(fake);
    uint8_t* const fb = static_cast<uint8_t*>(fake);
    uint64_t* const fl = static_cast<uint64_t*>(fake);
    int* const fs = static_cast<int*>(fake);
    CHECK(tlc_compress(ff, ff, 0, 1.5f, fb, 10, fl, ff, ws, 4096, fs, nullptr) == TLC_ERR_INVALID_ARG);
    CHECK(tlc_compress(ff, ff, 11, 1.5f, fb, 2, fl, ff, ws, 4096, fs, nullptr) == TLC_ERR_CAPACITY);
    CHECK(tlc_compress(static_cast<float*>(odd), ff, 10, 1.5f, fb, 10, fl, ff, ws, 4096, fs, nullptr) ==
          TLC_ERR_INVALID_ARG);
    CHECK(tlc_compress(ff, ff, 10, 0.5f, fb, 10, fl, ff, ws, 4096, fs, nullptr) == TLC_ERR_INVALID_ARG);
    CHECK(tlc_compress(ff, ff, 10, 1.5f, fb, 10, fl, ff, nullptr, 4096, fs, nullptr) == TLC_ERR_WORKSPACE);
    CHECK(tlc_compress_static(ff, ff, tlc_compress_static_max_n() + 1, 1.5f, fb, 1ull << 40, fl, ff, fs,
                              nullptr) == TLC_ERR_TOO_LARGE);
    CHECK(tlc_decompress(fb, fl, ff, 0, 1.5f, ff, ws, 4096, fs, nullptr, nullptr) == TLC_ERR_INVALID_ARG);
    CHECK(tlc_decompress(fb, nullptr, ff, 10, 1.5f, ff, ws, 4096, fs, nullptr, nullptr) == TLC_ERR_INVALID_ARG);
    CHECK(tlc_decompress_accumulate(fb, fl, ff, 10, 1.99f, ff, ws, 1, fs, nullptr) == TLC_ERR_WORKSPACE);
    CHECK(tlc_server_compress(ff, 0, ff, 10, 1.5f, fb, 10, fl, ff, ws, 4096, fs, nullptr) == TLC_ERR_INVALID_ARG);
    CHECK(tlc_copy_probe(fake, fake, 17, nullptr) == TLC_ERR_INVALID_ARG);
    const uint64_t two[] = {100, 200};
    tlc_group_info g{};
    CHECK(tlc_group_plan(two, 2, &g, nullptr, 0, nullptr) == TLC_OK);
    tlc_group_info bad = g;
    bad.table_bytes += 16;
    CHECK(tlc_compress_group(&bad, fake, ff, ff, 1.5f, fb, fl, ff, ws, 1 << 20, fs, nullptr) == TLC_ERR_INVALID_ARG);
    CHECK(tlc_compress_group(&g, nullptr, ff, ff, 1.5f, fb, fl, ff, ws, 1 << 20, fs, nullptr) == TLC_ERR_INVALID_ARG);
    CHECK(tlc_compress_group(nullptr, fake, ff, ff, 1.5f, fb, fl, ff, ws, 1 << 20, fs, nullptr) ==
          TLC_ERR_INVALID_ARG);
    CHECK(tlc_decompress_group(&g, fake, fb, fl, ff, 1.5f, ff, ws, 16, fs, nullptr, nullptr) == TLC_ERR_WORKSPACE);
    CHECK(tlc_decompress_accumulate_many_group(&g, fake, 0, fb, g.stream_bytes, fl, ff, 1.5f, ff, ws, 1 << 20, fs,
                                               nullptr, nullptr) == TLC_ERR_INVALID_ARG);
    CHECK(tlc_decompress_accumulate_many_group(&g, fake, 2, fb, g.stream_bytes - 16, fl, ff, 1.5f, ff, ws, 1 << 20,
                                               fs, nullptr, nullptr) == TLC_ERR_INVALID_ARG);
    CHECK(tlc_decompress_accumulate_many_group(&g, fake, 2, fb, g.stream_bytes, fl, ff, 1.5f, ff, ws, 16, fs,
                                               nullptr, nullptr) == TLC_ERR_WORKSPACE);
    {
        tlc_group_info huge = g;  // unit ids of payloads x tensors must stay below 2^31
        huge.count = 1ull << 26;
        huge.chunks = 1ull << 26;
        CHECK(tlc_accumulate_many_workspace_size(&huge, 31) > 0);
        CHECK(tlc_accumulate_many_workspace_size(&huge, 32) == 0);
    }
    {
        const uint64_t bound = tlc_wire_bound(&g), ww = tlc_wire_workspace_size(&g);
        CHECK(tlc_wire_pack_group(&g, fake, fb, fl, ff, fb, bound - 1, fl, ws, ww, fs, nullptr) == TLC_ERR_CAPACITY);
        CHECK(tlc_wire_pack_group(&g, fake, fb, fl, ff, fb, bound, fl, ws, ww - 1, fs, nullptr) == TLC_ERR_WORKSPACE);
        CHECK(tlc_wire_pack_group(&g, fake, nullptr, fl, ff, fb, bound, fl, ws, ww, fs, nullptr) ==
              TLC_ERR_INVALID_ARG);
        CHECK(tlc_wire_pack_group(&bad, fake, fb, fl, ff, fb, bound, fl, ws, ww, fs, nullptr) == TLC_ERR_INVALID_ARG);
        CHECK(tlc_wire_unpack_group(&g, fake, fb, 8 * g.count - 1, fb, fl, ff, ws, ww, fs, nullptr) ==
              TLC_ERR_CAPACITY);
        CHECK(tlc_wire_unpack_group(&g, fake, fb, 8 * g.count, fb, fl, ff, nullptr, ww, fs, nullptr) ==
              TLC_ERR_WORKSPACE);
        CHECK(tlc_wire_unpack_group(&g, fake, fb, 8 * g.count, fb, fl, nullptr, ws, ww, fs, nullptr) ==
              TLC_ERR_INVALID_ARG);
        CHECK(tlc_wire_bound(nullptr) == 0 && tlc_wire_workspace_size(nullptr) == 0);
        const uint32_t cuts_ok[2] = {0, (uint32_t)g.count}, cuts_bad[2] = {0, (uint32_t)g.count + 1};
        CHECK(tlc_wire_unpack_ranges_group(&g, fake, nullptr, 1, fb, 8 * g.count, fb, fl, ff, ws, ww, fs, nullptr) ==
              TLC_ERR_INVALID_ARG);
        CHECK(tlc_wire_unpack_ranges_group(&g, fake, cuts_bad, 1, fb, 8 * g.count, fb, fl, ff, ws, ww, fs,
                                           nullptr) == TLC_ERR_INVALID_ARG);
        CHECK(tlc_wire_unpack_ranges_group(&g, fake, cuts_ok, 1, fb, 8 * g.count - 1, fb, fl, ff, ws, ww, fs,
                                           nullptr) == TLC_ERR_CAPACITY);
    }
    CHECK(tlc_planes_gather(ff, fl, ff, fl, nullptr, 3, 100, nullptr) == TLC_ERR_INVALID_ARG);
    CHECK(tlc_planes_scatter(ff, fl, ff, fl, fl, 65536, 100, nullptr) == TLC_ERR_INVALID_ARG);

    if (failures) {
        std::fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    std::printf("host checks ok\n");
    return 0;
}
