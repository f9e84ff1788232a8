// Host sanitizer run of the C-ABI validation (kda_api.cpp built with
// AddressSanitizer and UndefinedBehaviorSanitizer for the host by
// tests/test_sanitizers.py). Every call below is rejected, or is a no-op or
// a size query, before any HIP call, so it runs without a GPU. Exit status 0
// = every status as expected (the sanitizers abort on their own findings).
#include <climits>
#include <cstdint>
#include <cstdio>

#include "kda.h"

static int fails = 0;
static void expect(const char* what, int got, int want) {
    if (got != want) {
        std::printf("FAIL %s: status %d, expected %d\n", what, got, want);
        ++fails;
    }
}

int main() {
    char* base = reinterpret_cast<char*>(uintptr_t(1) << 40);   // never dereferenced
    auto P = [&](int i, int off = 0) { return static_cast<void*>(base + (size_t(i) << 30) + off); };
    float* F = nullptr;
    const int INV = KDA_ERR_INVALID_ARG, UNS = KDA_ERR_UNSUPPORTED, WS = KDA_ERR_WORKSPACE;

    // size queries: huge and negative sizes must not overflow
    std::printf("ws %zu %zu %zu\n", kda_prefill_workspace_size(INT_MAX, INT_MAX, INT_MAX, 128, 128, KDA_BF16, 64),
                kda_prefill_workspace_size(-1, 10, 1, 128, 128, KDA_BF16, 64),
                kda_prefill_varlen_workspace_size(INT_MAX, INT_MAX, INT_MAX, 128, 128, KDA_BF16, 64));
    expect("varlen ws negative", (int)kda_prefill_varlen_workspace_size(-3, 5, 1, 128, 128, KDA_BF16, 64), 0);

    // prefill
    expect("prefill huge", kda_prefill_fwd(P(0), P(1), P(2), (float*)P(3), (float*)P(4), F, P(6), F,
                                           INT_MAX, INT_MAX, INT_MAX, 128, 128, KDA_BF16, 64, P(10), SIZE_MAX, nullptr), INV);
    expect("prefill negative", kda_prefill_fwd(P(0), P(1), P(2), (float*)P(3), (float*)P(4), F, P(6), F,
                                               1, -1, 1, 128, 128, KDA_BF16, 64, P(10), 1 << 20, nullptr), INV);
    expect("prefill dk", kda_prefill_fwd(P(0), P(1), P(2), (float*)P(3), (float*)P(4), F, P(6), F,
                                         1, 64, 2, 48, 128, KDA_BF16, 64, P(10), 1 << 20, nullptr), UNS);
    expect("prefill misaligned", kda_prefill_fwd(P(0, 2), P(1), P(2), (float*)P(3), (float*)P(4), F, P(6), F,
                                                 1, 64, 2, 128, 128, KDA_BF16, 64, P(10), SIZE_MAX, nullptr), INV);
    expect("prefill overlap", kda_prefill_fwd(P(0), P(1), P(2), (float*)P(3), (float*)P(4), F, P(0, 256), F,
                                              1, 64, 2, 128, 128, KDA_BF16, 64, P(10), SIZE_MAX, nullptr), INV);
    expect("prefill no ws", kda_prefill_fwd(P(0), P(1), P(2), (float*)P(3), (float*)P(4), F, P(6), F,
                                            1, 64, 2, 128, 128, KDA_BF16, 64, nullptr, 0, nullptr), WS);
    expect("prefill empty", kda_prefill_fwd(nullptr, nullptr, nullptr, F, F, F, nullptr, F,
                                            0, 64, 2, 128, 128, KDA_BF16, 64, nullptr, 0, nullptr), KDA_OK);

    // varlen
    expect("varlen huge", kda_prefill_varlen(P(0), P(1), P(2), (float*)P(3), (float*)P(4), F, P(6), F, (int*)P(8),
                                             INT_MAX, INT_MAX, INT_MAX, 128, 128, KDA_BF16, 64, (float*)P(9), 64, INT_MAX,
                                             P(10), SIZE_MAX, nullptr), INV);
    expect("varlen ckpt", kda_prefill_varlen(P(0), P(1), P(2), (float*)P(3), (float*)P(4), F, P(6), F, (int*)P(8),
                                             3, 300, 2, 128, 128, KDA_BF16, 64, (float*)P(9), 100, 4,
                                             P(10), SIZE_MAX, nullptr), INV);
    expect("varlen cu", kda_prefill_varlen(P(0), P(1), P(2), (float*)P(3), (float*)P(4), F, P(6), F, nullptr,
                                           3, 300, 2, 128, 128, KDA_BF16, 64, (float*)P(9), 64, 4,
                                           P(10), SIZE_MAX, nullptr), INV);
    expect("varlen empty", kda_prefill_varlen(nullptr, nullptr, nullptr, F, F, F, nullptr, F, nullptr,
                                              0, 0, 2, 128, 128, KDA_BF16, 64, nullptr, 0, 0, nullptr, 0, nullptr), KDA_OK);

    // decode, multi-token decode
    expect("decode huge", kda_decode_step(P(0), P(1), P(2), (float*)P(3), (float*)P(4), (float*)P(5), P(6),
                                          INT_MAX, INT_MAX, 128, 128, KDA_BF16, nullptr), INV);
    expect("decode null", kda_decode_step(nullptr, P(1), P(2), (float*)P(3), (float*)P(4), (float*)P(5), P(6),
                                          2, 2, 128, 128, KDA_BF16, nullptr), INV);
    expect("multi huge", kda_decode_multi(P(0), P(1), P(2), (float*)P(3), (float*)P(4), (float*)P(5), P(6),
                                          (int*)P(7), INT_MAX, INT_MAX, INT_MAX, 128, 128, KDA_BF16, nullptr), INV);
    expect("multi n misaligned", kda_decode_multi(P(0), P(1), P(2), (float*)P(3), (float*)P(4), (float*)P(5), P(6),
                                                  (int*)P(7, 2), 2, 4, 2, 128, 128, KDA_BF16, nullptr), INV);

    // layer form
    kda_layer_opts bad{};
    bad.gate = (kda_gate)3;   // no such mode (3 is inside the enum's value range)
    expect("layer gate", kda_prefill_layer(P(0), P(1), P(2), P(3), (float*)P(4), F, P(6), F, 1, 64, 2, 128, 128,
                                           KDA_BF16, 64, &bad, P(10), SIZE_MAX, nullptr), INV);
    kda_layer_opts huge{};
    expect("layer huge", kda_prefill_layer(P(0), P(1), P(2), P(3), (float*)P(4), F, P(6), F, INT_MAX, INT_MAX,
                                           INT_MAX, 128, 128, KDA_BF16, 64, &huge, P(10), SIZE_MAX, nullptr), INV);
    expect("layer decode overlap", kda_decode_layer(P(0), P(1), P(2), P(3), (float*)P(4), (float*)P(3, 256), P(6),
                                                    2, 2, 128, 128, KDA_BF16, nullptr, nullptr), INV);

    for (int s = 0; s <= 7; ++s) std::printf("status %d: %s\n", s, kda_status_string((kda_status)s));
    std::printf("%d failures\n", fails);
    return fails != 0;
}
