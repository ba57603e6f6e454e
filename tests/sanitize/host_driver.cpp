// Host sanitizer run of the library's host-only protocol code (test
// infrastructure): afd_layout_compute over valid and invalid configurations,
// the header codec (round trips, bad magic / version / counts, the largest
// expert count), the inbound message checks and field sizes of afd_proto.h,
// status strings, and the argument checks of the entry points that refuse
// before touching a device.  Linked against afd_host.cpp with the kernel
// launches stubbed out (sanitize/launch_stubs.cpp); built with
// AddressSanitizer and UndefinedBehaviorSanitizer on the host side by
// tests/test_sanitize_cpu.py.  Exit 0 and no report is a pass.
#include <cstdio>
#include <cstring>
#include <vector>

#include "afd.h"
#include "../../combine_afd_slot_amd/csrc/afd_proto.h"

static afd_window_config cfg(int P, int R, int cap, int H, int E, int K, int I, int Is) {
    afd_window_config c;
    std::memset(&c, 0, sizeof c);
    c.struct_size = sizeof c;
    c.num_peers = P;
    c.ring_depth = R;
    c.token_cap = cap;
    c.hidden = H;
    c.num_experts = E;
    c.top_k = K;
    c.intermediate = I;
    c.shared_intermediate = Is;
    c.routed_scaling_factor = 1.0f;
    c.renormalize = 1;
    c.poll_timeout_us = 1000;
    return c;
}

int main() {
    int fails = 0;
    afd_layout L;
    // valid layouts, including the limits (64 peers, ring 4, 1024 experts, top-16)
    const afd_window_config ok[] = {cfg(2, 1, 16, 64, 8, 2, 32, 32), cfg(8, 1, 16, 2048, 64, 6, 1408, 2816),
                                    cfg(64, 4, 33, 256, 1024, 16, 128, 0), cfg(2, 2, 4096, 7168, 256, 8, 2048, 2048),
                                    cfg(1, 1, 1, 8, 1, 1, 8, 8)};
    for (const auto& c : ok) {
        if (afd_layout_compute(&c, &L) != AFD_OK) ++fails;
        if (L.total_bytes <= 0 || L.slot_bytes % 256 || L.workspace_off % 256) ++fails;
        for (int f = 0; f < AFD_NUM_FIELDS; ++f)
            if (L.field_off[f] % 256 || L.field_off[f] + L.field_bytes[f] > L.slot_bytes) ++fails;
    }
    afd_window_config v = cfg(2, 1, 16, 64, 8, 2, 32, 32);
    v.attention_routes = 1;
    if (afd_layout_compute(&v, &L) != AFD_OK) ++fails;
    v.route_experts = 16;
    v.expert_offset = 8;
    if (afd_layout_compute(&v, &L) != AFD_OK) ++fails;
    // invalid ones are refused
    std::vector<afd_window_config> bad;
    for (int i = 0; i < 14; ++i) bad.push_back(cfg(2, 1, 16, 64, 8, 2, 32, 32));
    bad[0].struct_size = 4;
    bad[1].num_peers = 0;
    bad[2].num_peers = 65;
    bad[3].ring_depth = 5;
    bad[4].token_cap = 0;
    bad[5].hidden = 60;  // not a multiple of 8
    bad[6].top_k = 9;    // > num_experts
    bad[7].num_experts = 1025;
    bad[8].renormalize = 2;
    bad[9].poll_timeout_us = 0;
    bad[10].reserved[0] = 1;
    bad[11].expert_offset = 1;  // without route_experts
    bad[12].route_experts = 16;  // without attention_routes
    bad[13].w1_fp8 = 1;          // hidden 64 is fine, but top_k ... keep valid
    bad[13].hidden = 72;         // fp8 needs hidden a multiple of 64
    for (auto& c : bad)
        if (afd_layout_compute(&c, &L) == AFD_OK) ++fails;
    if (afd_layout_compute(nullptr, &L) == AFD_OK) ++fails;
    // header codec
    std::vector<int32_t> counts(1024), words(12 + 1024);
    for (int i = 0; i < 1024; ++i) counts[i] = i * 7 - 3;
    afd_header_fields f{0x2, 41, 40, 3, 1, 77, 77 * 8, 77, 5, 1024}, g;
    if (afd_header_encode(&f, counts.data(), words.data()) != AFD_OK) ++fails;
    if (afd_header_decode(words.data(), (int32_t)words.size(), 1024, &g) != AFD_OK) ++fails;
    if (std::memcmp(&f, &g, sizeof f) != 0) ++fails;
    for (int i = 0; i < 1024; ++i)
        if (words[12 + i] != counts[i]) ++fails;
    if (afd_header_decode(words.data(), (int32_t)words.size(), 1023, &g) == AFD_OK) ++fails;
    if (afd_header_decode(words.data(), 11, 1024, &g) == AFD_OK) ++fails;  // shorter than the fixed words
    words[AFD_HDR_MAGIC] ^= 1;
    if (afd_header_decode(words.data(), (int32_t)words.size(), 1024, &g) == AFD_OK) ++fails;
    words[AFD_HDR_MAGIC] ^= 1;
    words[AFD_HDR_VERSION] = 2;
    if (afd_header_decode(words.data(), (int32_t)words.size(), 1024, &g) == AFD_OK) ++fails;
    // inbound checks and field sizes of the device/host protocol header
    afd_header_fields h{0, 9, 0, 2, 1, 10, 10, 10, 3, 8};
    if (afd::inbound_check(h, 3, 1, 2, 16, 9, true, 1, false) != AFD_OK) ++fails;
    if (afd::inbound_check(h, 3, 1, 2, 16, 8, true, 1, false) == AFD_OK) ++fails;   // stale seq
    if (afd::inbound_check(h, 3, 1, 2, 9, 9, true, 1, false) == AFD_OK) ++fails;    // over capacity
    if (afd::inbound_check(h, 3, 1, 2, 16, 9, false, 1, false) == AFD_OK) ++fails;  // shared rows in a routed-only window
    int64_t fb[AFD_NUM_FIELDS];
    afd::slot_field_bytes(16, 64, 8, 2, true, false, fb);
    if (fb[AFD_FIELD_ROUTED_X] != 2 * 16 * 64 || fb[AFD_FIELD_SHARED_X] != 2 * 16 * 64) ++fails;
    afd::slot_field_bytes(16, 64, 8, 2, false, true, fb);
    if (fb[AFD_FIELD_ROUTE_TABLE] != 0 || fb[AFD_FIELD_ROUTED_X] != 2 * 16 * 2 * 64 || fb[AFD_FIELD_SHARED_X]) ++fails;
    // refusals before any device work
    for (int s = -9; s <= 1; ++s)
        if (!afd_status_string(s)) ++fails;
    if (afd_window_destroy(nullptr) != AFD_OK) ++fails;
    afd_window* w = nullptr;
    afd_window_config huge = cfg(2, 1, 4096, 2048, 64, 6, 1408, 2816);
    if (afd_window_create_static(&huge, &w) != AFD_ERR_CAPACITY || w) ++fails;
    if (afd_window_create(&bad[1], &w) == AFD_OK || w) ++fails;
    if (afd_slot_pack(nullptr, 0, 0, 0, 0, nullptr, nullptr, 0, nullptr) == AFD_OK) ++fails;
    if (afd_ffn_run(nullptr, 0, 0, nullptr, nullptr) == AFD_OK) ++fails;
    if (std::strlen(afd_last_error()) == 0) ++fails;
    if (afd_abi_version() != AFD_ABI_VERSION) ++fails;
    std::printf("host sanitizer driver: %d failure(s)\n", fails);
    return fails ? 1 : 0;
}
