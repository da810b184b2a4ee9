// Drives every entry point of include/la_chunk.h through its host-side validation, built with
// AddressSanitizer against stand-in launchers (stub_launchers.cpp): accepted calls must reach
// the launcher the dispatch rules name, rejected ones must return their status and launch
// nothing.  Device pointers are fake, aligned, non-overlapping addresses: the validation only
// compares and offsets them, it never dereferences them.  Exit status 0 when every case holds.
#include <stdint.h>
#include <stdio.h>

#include "la_chunk.h"

extern int g_last_launch;
enum {
    L_NONE = 0, L_FWD, L_BWD, L_FWD_C128, L_BWD_C128, L_SEQ_FWD_C128, L_SEQ_BWD_C128, L_SEQ_FWD_D128,
    L_SEQ_BWD_D128, L_CE_FWD, L_CE_BWD, L_CE_FWD_NOALLOC, L_FLOOR, L_CUMSUM_FWD, L_CUMSUM_BWD, L_BWD_D128
};

static int failures = 0;

static void *A(int i) { return reinterpret_cast<void *>((uintptr_t)1 << 40 | (uintptr_t)i << 32); }
static float *F(int i) { return static_cast<float *>(A(i)); }

static void expect(const char *what, la_status got, la_status want, int launch_want) {
    const int launched = g_last_launch;
    g_last_launch = L_NONE;
    if (got != want || launched != (want == LA_OK ? launch_want : L_NONE)) {
        printf("FAIL %s: status %d (want %d), launcher %d (want %d)\n", what, (int)got, (int)want, launched,
               want == LA_OK ? launch_want : L_NONE);
        ++failures;
    }
}

int main() {
    // ---- la_chunk_fwd
    expect("fwd headline", la_chunk_fwd(A(0), A(1), A(2), F(3), F(4), A(5), F(6), F(7), 160, 128, 64, 64, LA_FEATURE_NONE, LA_BF16, 0),
           LA_OK, L_FWD_C128);
    expect("fwd ragged", la_chunk_fwd(A(0), A(1), A(2), F(3), F(4), A(5), F(6), F(7), 4, 100, 64, 64, LA_FEATURE_NONE, LA_BF16, 0),
           LA_OK, L_FWD);
    expect("fwd bf16 d128 ragged: the D = 128 sequence forward",
           la_chunk_fwd(A(0), A(1), A(2), F(3), F(4), A(5), F(6), F(7), 4, 100, 128, 64, LA_FEATURE_NONE, LA_BF16, 0),
           LA_OK, L_SEQ_FWD_D128);
    expect("fwd bf16 d128 beyond the sequence kernel's length",
           la_chunk_fwd(A(0), A(1), A(2), F(3), F(4), A(5), F(6), F(7), 1, LA_SEQ_D128_MAX_T + 1, 128, 64, LA_FEATURE_NONE,
                        LA_BF16, 0),
           LA_OK, L_FWD);
    expect("fwd fp32 d128 no carry",
           la_chunk_fwd(A(0), A(1), A(2), nullptr, nullptr, A(5), F(6), F(7), 1, 37, 128, 64, LA_FEATURE_NONE, LA_F32, 0), LA_OK, L_FWD);
    expect("fwd G=0", la_chunk_fwd(A(0), A(1), A(2), F(3), F(4), A(5), F(6), F(7), 0, 128, 64, 64, LA_FEATURE_NONE, LA_BF16, 0),
           LA_ERR_INVALID, 0);
    expect("fwd D=96", la_chunk_fwd(A(0), A(1), A(2), F(3), F(4), A(5), F(6), F(7), 4, 128, 96, 64, LA_FEATURE_NONE, LA_BF16, 0),
           LA_ERR_UNSUPPORTED, 0);
    expect("fwd half carry", la_chunk_fwd(A(0), A(1), A(2), nullptr, F(4), A(5), F(6), F(7), 4, 128, 64, 64, LA_FEATURE_NONE, LA_BF16, 0),
           LA_ERR_INVALID, 0);
    expect("fwd misaligned",
           la_chunk_fwd((char *)A(0) + 8, A(1), A(2), F(3), F(4), A(5), F(6), F(7), 4, 128, 64, 64, LA_FEATURE_NONE, LA_BF16, 0),
           LA_ERR_ALIGN, 0);
    expect("fwd S_out == S_in", la_chunk_fwd(A(0), A(1), A(2), F(3), F(4), A(5), F(3), F(7), 4, 128, 64, 64, LA_FEATURE_NONE, LA_BF16, 0),
           LA_ERR_ALIAS, 0);
    expect("fwd overflow",
           la_chunk_fwd(A(0), A(1), A(2), F(3), F(4), A(5), F(6), F(7), 0x7fffffff, 0x7fffffff, 128, 64, LA_FEATURE_NONE, LA_BF16, 0),
           LA_ERR_INVALID, 0);

    // ---- la_chunk_bwd
    expect("bwd headline",
           la_chunk_bwd(A(0), A(1), A(2), F(3), F(4), A(5), nullptr, nullptr, A(8), A(9), A(10), F(11), F(12), 160, 128,
                        64, 64, LA_FEATURE_NONE, LA_BF16, 0),
           LA_OK, L_BWD_C128);
    expect("bwd d128 upstream",
           la_chunk_bwd(A(0), A(1), A(2), F(3), F(4), A(5), F(6), F(7), A(8), A(9), A(10), F(11), F(12), 160, 100, 128,
                        64, LA_FEATURE_NONE, LA_BF16, 0),
           LA_OK, L_BWD_D128);
    expect("bwd fp32 d64",
           la_chunk_bwd(A(0), A(1), A(2), F(3), F(4), A(5), F(6), F(7), A(8), A(9), A(10), F(11), F(12), 16, 100, 64,
                        64, LA_FEATURE_NONE, LA_F32, 0),
           LA_OK, L_BWD);
    expect("bwd C > max",
           la_chunk_bwd(A(0), A(1), A(2), F(3), F(4), A(5), F(6), F(7), A(8), A(9), A(10), F(11), F(12), 4,
                        LA_BWD_MAX_C + 1, 64, 64, LA_FEATURE_NONE, LA_BF16, 0),
           LA_ERR_UNSUPPORTED, 0);
    expect("bwd dq == dO",
           la_chunk_bwd(A(0), A(1), A(2), F(3), F(4), A(5), F(6), F(7), A(5), A(9), A(10), F(11), F(12), 4, 128, 64, 64,
                        LA_FEATURE_NONE, LA_BF16, 0),
           LA_ERR_ALIAS, 0);
    expect("bwd half upstream",
           la_chunk_bwd(A(0), A(1), A(2), F(3), F(4), A(5), F(6), nullptr, A(8), A(9), A(10), F(11), F(12), 4, 128, 64,
                        64, LA_FEATURE_NONE, LA_BF16, 0),
           LA_ERR_INVALID, 0);

    // ---- block 1 (the cumsum form), the fused feature map, the fp32 backward at D = 128
    expect("fwd cumsum", la_chunk_fwd(A(0), A(1), A(2), F(3), F(4), A(5), F(6), F(7), 160, 128, 64, 1,
                                      LA_FEATURE_NONE, LA_BF16, 0),
           LA_OK, L_CUMSUM_FWD);
    expect("fwd elu1 headline", la_chunk_fwd(A(0), A(1), A(2), F(3), F(4), A(5), F(6), F(7), 160, 128, 64, 64,
                                             LA_FEATURE_ELU1, LA_BF16, 0),
           LA_OK, L_FWD_C128);
    expect("fwd elu1 ragged", la_chunk_fwd(A(0), A(1), A(2), F(3), F(4), A(5), F(6), F(7), 160, 100, 64, 64,
                                           LA_FEATURE_ELU1, LA_BF16, 0),
           LA_OK, L_CUMSUM_FWD);
    expect("fwd bad feature", la_chunk_fwd(A(0), A(1), A(2), F(3), F(4), A(5), F(6), F(7), 160, 100, 64, 64,
                                           (la_feature)9, LA_BF16, 0),
           LA_ERR_INVALID, 0);
    expect("bwd fp32 d128", la_chunk_bwd(A(0), A(1), A(2), F(3), F(4), A(5), F(6), F(7), A(8), A(9), A(10), F(11),
                                         F(12), 160, 128, 128, 64, LA_FEATURE_NONE, LA_F32, 0),
           LA_OK, L_CUMSUM_BWD);
    expect("bwd cumsum ragged", la_chunk_bwd(A(0), A(1), A(2), nullptr, nullptr, A(5), nullptr, nullptr, A(8), A(9),
                                             A(10), F(11), F(12), 3, 37, 64, 1, LA_FEATURE_ELU1, LA_BF16, 0),
           LA_OK, L_CUMSUM_BWD);
    expect("bwd elu1 headline", la_chunk_bwd(A(0), A(1), A(2), F(3), F(4), A(5), nullptr, nullptr, A(8), A(9), A(10),
                                             F(11), F(12), 160, 128, 64, 64, LA_FEATURE_ELU1, LA_BF16, 0),
           LA_OK, L_BWD_C128);
    expect("seq block 1", la_seq_fwd(A(0), A(1), A(2), F(3), F(4), A(5), F(6), F(7), F(8), F(9), 4, 512, 64, 128, 1,
                                     LA_FEATURE_NONE, LA_BF16, 0),
           LA_ERR_UNSUPPORTED, 0);

    // ---- sequence calls
    expect("seq fwd d64",
           la_seq_fwd(A(0), A(1), A(2), F(3), F(4), A(5), F(6), F(7), F(8), F(9), 1280, 1024, 64, 128, 64,
                      LA_FEATURE_NONE, LA_BF16, 0),
           LA_OK, L_SEQ_FWD_C128);
    expect("seq fwd d128 ragged elu1",
           la_seq_fwd(A(0), A(1), A(2), F(3), F(4), A(5), F(6), F(7), nullptr, nullptr, 160, 8164, 128, 128, 64,
                      LA_FEATURE_ELU1, LA_BF16, 0),
           LA_OK, L_SEQ_FWD_D128);
    expect("seq fwd d64 partial chunk",
           la_seq_fwd(A(0), A(1), A(2), F(3), F(4), A(5), F(6), F(7), F(8), F(9), 4, 500, 64, 128, 64, LA_FEATURE_NONE,
                      LA_BF16, 0),
           LA_ERR_UNSUPPORTED, 0);
    expect("seq fwd bad feature",
           la_seq_fwd(A(0), A(1), A(2), F(3), F(4), A(5), F(6), F(7), F(8), F(9), 4, 512, 64, 128, 64, (la_feature)5,
                      LA_BF16, 0),
           LA_ERR_INVALID, 0);
    expect("seq bwd d64",
           la_seq_bwd(A(0), A(1), A(2), F(3), F(4), F(5), F(6), A(7), nullptr, nullptr, A(10), A(11), A(12), F(13),
                      F(14), 1280, 1024, 64, 128, 64, LA_FEATURE_NONE, LA_BF16, 0),
           LA_OK, L_SEQ_BWD_C128);
    expect("seq bwd d128",
           la_seq_bwd(A(0), A(1), A(2), F(3), F(4), nullptr, nullptr, A(7), F(8), F(9), A(10), A(11), A(12), F(13),
                      F(14), 160, 8164, 128, 128, 64, LA_FEATURE_NONE, LA_BF16, 0),
           LA_OK, L_SEQ_BWD_D128);
    expect("seq bwd no final carry",
           la_seq_bwd(A(0), A(1), A(2), nullptr, F(4), nullptr, nullptr, A(7), nullptr, nullptr, A(10), A(11), A(12),
                      F(13), F(14), 4, 512, 64, 128, 64, LA_FEATURE_NONE, LA_BF16, 0),
           LA_ERR_INVALID, 0);

    // ---- cross-entropy
    const size_t fws = la_ce_fwd_workspace_bytes(512, 1280, 50257);
    const size_t bws = la_ce_workspace_bytes(512, 1280, 50257, 128);
    if (fws == 0 || bws < fws) {
        printf("FAIL workspace sizes %zu %zu\n", fws, bws);
        ++failures;
    }
    expect("ce fwd", la_ce_fwd(A(0), A(1), (const int *)A(2), F(3), F(4), A(5), fws, 512, 1280, 50257, LA_BF16, 0),
           LA_OK, L_CE_FWD);
    expect("ce fwd small ws",
           la_ce_fwd(A(0), A(1), (const int *)A(2), F(3), F(4), A(5), fws - 1, 512, 1280, 50257, LA_BF16, 0),
           LA_ERR_INVALID, 0);
    expect("ce bwd chunked",
           la_ce_bwd(A(0), A(1), (const int *)A(2), F(3), nullptr, A(5), F(6), A(7), bws, 512, 1280, 50257, 128,
                     LA_BF16, 0),
           LA_OK, L_CE_BWD);
    expect("ce bwd d=100",
           la_ce_bwd(A(0), A(1), (const int *)A(2), F(3), nullptr, A(5), F(6), A(7), bws, 512, 100, 50257, 128,
                     LA_BF16, 0),
           LA_ERR_UNSUPPORTED, 0);

    expect("ce fwd noalloc", la_ce_fwd_noalloc(A(0), A(1), (const int *)A(2), F(3), F(4), 512, 1280, 50257, LA_BF16, 0),
           LA_OK, L_CE_FWD_NOALLOC);
    expect("ce fwd noalloc beyond scratch",
           la_ce_fwd_noalloc(A(0), A(1), (const int *)A(2), F(3), F(4), 6000, 128, 50257, LA_BF16, 0),
           LA_ERR_UNSUPPORTED, 0);

    // ---- launch floors
    expect("floor empty", la_floor_launch(0, 160, nullptr, 0, A(1), 2048, 0), LA_OK, L_FLOOR);
    expect("floor fwd", la_floor_launch(1, 160, A(0), 160 * 65536, A(1), 160 * 32768, 0), LA_OK, L_FLOOR);
    expect("floor bwd small out", la_floor_launch(2, 160, A(0), 160 * 81920, A(1), 160 * 65536 - 1, 0),
           LA_ERR_INVALID, 0);
    expect("floor bwd, 128-thread workgroups", la_floor_launch(4, 640, A(0), 640 * 20480, A(1), 640 * 16384, 0),
           LA_OK, L_FLOOR);
    expect("floor fwd, 128-thread workgroups, small in",
           la_floor_launch(3, 640, A(0), 640 * 16384 - 1, A(1), 640 * 8192, 0), LA_ERR_INVALID, 0);
    expect("floor bad kind", la_floor_launch(5, 160, A(0), 1 << 30, A(1), 1 << 30, 0), LA_ERR_INVALID, 0);
    expect("floor overlap", la_floor_launch(1, 160, A(0), 160 * 65536, (char *)A(0) + 4096, 160 * 32768, 0),
           LA_ERR_ALIAS, 0);

    // ---- the rest of the boundary
    for (int s = -1; s <= 6; ++s)
        if (la_status_str((la_status)s) == nullptr) {
            printf("FAIL la_status_str(%d) is NULL\n", s);
            ++failures;
        }
    if (la_abi_version() != LA_ABI_VERSION) {
        printf("FAIL la_abi_version\n");
        ++failures;
    }
    if (la_time_next_launch(A(0), nullptr) != LA_ERR_INVALID || la_time_next_launch(nullptr, nullptr) != LA_OK) {
        printf("FAIL la_time_next_launch\n");
        ++failures;
    }
    if (!la_kernel_name(1, LA_BF16, 128, 64, 64, LA_FEATURE_NONE) || la_kernel_name(1, LA_F32, 128, 96, 64, LA_FEATURE_NONE) ||
        !la_seq_kernel_name(0, LA_BF16, 128, 128, LA_FEATURE_ELU1))
        ++failures;

    printf("%s: %d failures\n", failures ? "FAILED" : "ok", failures);
    return failures ? 1 : 0;
}
