// Host-only stand-ins for the library's kernel launchers, so that the C ABI's argument
// validation (csrc/la_api.cpp) can be built with AddressSanitizer and run on a machine with
// no GPU.  Each stand-in records which launcher a call reached and launches nothing; the
// driver checks that every accepted call dispatches to the launcher the header's rules name.
#include <hip/hip_runtime.h>

#include "la_launch.h"

int g_last_launch = 0;  // which stand-in ran last (see the ids below)

namespace lachunk {

enum : int {
    L_FWD = 1, L_BWD, L_FWD_C128, L_BWD_C128, L_SEQ_FWD_C128, L_SEQ_BWD_C128, L_SEQ_FWD_D128, L_SEQ_BWD_D128,
    L_CE_FWD, L_CE_BWD, L_CE_FWD_NOALLOC, L_FLOOR, L_CUMSUM_FWD, L_CUMSUM_BWD, L_BWD_D128
};

static hipError_t hit(int id) {
    g_last_launch = id;
    return hipSuccess;
}

template <typename T, int D>
hipError_t launch_fwd(const void *, const void *, const void *, const float *, const float *, void *, float *,
                      float *, int, int, hipStream_t, const hipEvent_t *) {
    return hit(L_FWD);
}
template <typename T, int D>
hipError_t launch_bwd(const void *, const void *, const void *, const float *, const float *, const void *,
                      const float *, const float *, void *, void *, void *, float *, float *, int, int, hipStream_t,
                      const hipEvent_t *) {
    return hit(L_BWD);
}
template hipError_t launch_fwd<float, 64>(const void *, const void *, const void *, const float *, const float *,
                                          void *, float *, float *, int, int, hipStream_t, const hipEvent_t *);
template hipError_t launch_fwd<float, 128>(const void *, const void *, const void *, const float *, const float *,
                                           void *, float *, float *, int, int, hipStream_t, const hipEvent_t *);
template hipError_t launch_fwd<__bf16, 64>(const void *, const void *, const void *, const float *, const float *,
                                           void *, float *, float *, int, int, hipStream_t, const hipEvent_t *);
template hipError_t launch_fwd<__bf16, 128>(const void *, const void *, const void *, const float *, const float *,
                                            void *, float *, float *, int, int, hipStream_t, const hipEvent_t *);
template hipError_t launch_bwd<float, 64>(const void *, const void *, const void *, const float *, const float *,
                                          const void *, const float *, const float *, void *, void *, void *, float *,
                                          float *, int, int, hipStream_t, const hipEvent_t *);
template hipError_t launch_bwd<float, 128>(const void *, const void *, const void *, const float *, const float *,
                                           const void *, const float *, const float *, void *, void *, void *,
                                           float *, float *, int, int, hipStream_t, const hipEvent_t *);
template hipError_t launch_bwd<__bf16, 64>(const void *, const void *, const void *, const float *, const float *,
                                           const void *, const float *, const float *, void *, void *, void *,
                                           float *, float *, int, int, hipStream_t, const hipEvent_t *);
template hipError_t launch_bwd<__bf16, 128>(const void *, const void *, const void *, const float *, const float *,
                                            const void *, const float *, const float *, void *, void *, void *,
                                            float *, float *, int, int, hipStream_t, const hipEvent_t *);

hipError_t launch_fwd_c128(const void *, const void *, const void *, const float *, const float *, void *, float *,
                           float *, int, bool, hipStream_t, const hipEvent_t *) {
    return hit(L_FWD_C128);
}
hipError_t launch_bwd_c128(const void *, const void *, const void *, const float *, const float *, const void *,
                           const float *, const float *, void *, void *, void *, float *, float *, int, bool,
                           hipStream_t, const hipEvent_t *) {
    return hit(L_BWD_C128);
}
template <typename T, int D>
hipError_t launch_cumsum_fwd(const void *, const void *, const void *, const float *, const float *, void *, float *,
                             float *, int, int, bool, hipStream_t, const hipEvent_t *) {
    return hit(L_CUMSUM_FWD);
}
template <typename T, int D>
hipError_t launch_cumsum_bwd(const void *, const void *, const void *, const float *, const float *, const void *,
                             const float *, const float *, void *, void *, void *, float *, float *, int, int, bool,
                             hipStream_t, const hipEvent_t *) {
    return hit(L_CUMSUM_BWD);
}
#define STUB_CUMSUM(T, D)                                                                                          \
    template hipError_t launch_cumsum_fwd<T, D>(const void *, const void *, const void *, const float *,          \
                                                const float *, void *, float *, float *, int, int, bool,          \
                                                hipStream_t, const hipEvent_t *);                                  \
    template hipError_t launch_cumsum_bwd<T, D>(const void *, const void *, const void *, const float *,          \
                                                const float *, const void *, const float *, const float *, void *, \
                                                void *, void *, float *, float *, int, int, bool, hipStream_t,     \
                                                const hipEvent_t *);
STUB_CUMSUM(float, 64)
STUB_CUMSUM(float, 128)
STUB_CUMSUM(__bf16, 64)
STUB_CUMSUM(__bf16, 128)
hipError_t launch_seq_fwd_c128(const void *, const void *, const void *, const float *, const float *, void *,
                               float *, float *, float *, float *, int, int, bool, hipStream_t, const hipEvent_t *) {
    return hit(L_SEQ_FWD_C128);
}
hipError_t launch_seq_bwd_c128(const void *, const void *, const void *, const float *, const float *,
                               const float *, const float *, const void *, const float *, const float *, void *,
                               void *, void *, float *, float *, int, int, bool, hipStream_t, const hipEvent_t *) {
    return hit(L_SEQ_BWD_C128);
}
hipError_t launch_seq_fwd_d128(const void *, const void *, const void *, const float *, const float *, void *,
                               float *, float *, float *, float *, int, int, bool, hipStream_t, const hipEvent_t *) {
    return hit(L_SEQ_FWD_D128);
}
hipError_t launch_seq_bwd_d128(const void *, const void *, const void *, const float *, const float *,
                               const float *, const float *, const void *, const float *, const float *, void *,
                               void *, void *, float *, float *, int, int, bool, hipStream_t, const hipEvent_t *) {
    return hit(L_SEQ_BWD_D128);
}
hipError_t launch_bwd_d128(const void *, const void *, const void *, const float *, const float *, const void *,
                           const float *, const float *, void *, void *, void *, float *, float *, int, int, bool,
                           hipStream_t, const hipEvent_t *) {
    return hit(L_BWD_D128);
}
hipError_t launch_ce_fwd(const void *, const void *, const int *, float *, float *, void *, int, int, int,
                         hipStream_t, const hipEvent_t *) {
    return hit(L_CE_FWD);
}
hipError_t launch_ce_fwd_noalloc(const void *, const void *, const int *, float *, float *, int, int, int, hipStream_t,
                                 const hipEvent_t *) {
    return hit(L_CE_FWD_NOALLOC);
}
hipError_t launch_ce_bwd(const void *, const void *, const int *, const float *, const float *, void *, float *,
                         void *, int, int, int, int, hipStream_t, const hipEvent_t *) {
    return hit(L_CE_BWD);
}

hipError_t launch_floor(int, int, const void *, void *, hipStream_t, const hipEvent_t *) { return hit(L_FLOOR); }

}  // namespace lachunk
