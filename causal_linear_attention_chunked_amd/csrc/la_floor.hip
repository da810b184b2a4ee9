// Launch floors: kernels that do no arithmetic, to measure what one launch of a given size costs
// on the device apart from any computation.  An empty kernel, and streaming kernels of 512 (or
// 128) threads per workgroup that read and write the byte counts of the attention kernels'
// launches at the headline shape (160 groups, one 128-token chunk, D = 64, bf16; with 128 threads
// over four times the workgroups): every 16-byte load is
// issued before the first one is used (buffer loads), then the stores follow (non-temporal, as
// the one-chunk attention kernels store).  A measurement aid only: nothing on the attention or
// cross-entropy path calls these.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "la_launch.h"

namespace lachunk {

namespace {
typedef int int4v __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(FLOOR_THREADS) void la_floor_empty_kernel(int *flag, int never) {
    if (never) flag[threadIdx.x] = 1;  // never taken: the launch has a body the compiler keeps
}

template <int NIN, int NOUT, int NT>
__global__ __launch_bounds__(NT) void la_floor_stream_kernel(const int4v *__restrict__ in, int4v *__restrict__ out) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int4v *>(in + (size_t)blockIdx.x * NIN * NT), 0, NIN * NT * 16, 0x00020000);
    int4v x[NIN];
#pragma unroll
    for (int i = 0; i < NIN; ++i)
        x[i] = __builtin_bit_cast(int4v, __builtin_amdgcn_raw_buffer_load_b128(r, (threadIdx.x + NT * i) * 16, 0, 0));
    int4v acc = x[0];
#pragma unroll
    for (int i = 1; i < NIN; ++i) acc ^= x[i];
    int4v *dst = out + (size_t)blockIdx.x * NOUT * NT;
#pragma unroll
    for (int i = 0; i < NOUT; ++i) __builtin_nontemporal_store(acc + i, dst + threadIdx.x + NT * i);
}

template <int NIN, int NOUT, int NT>
void launch_stream(int nwg, const void *in, void *out, hipStream_t stream, const hipEvent_t ev[2]) {
    hipExtLaunchKernelGGL((la_floor_stream_kernel<NIN, NOUT, NT>), dim3((unsigned)nwg), dim3(NT), 0, stream, ev[0],
                          ev[1], 0, (const int4v *)in, (int4v *)out);
}
}  // namespace

hipError_t launch_floor(int kind, int nwg, const void *in, void *out, hipStream_t stream, const hipEvent_t ev[2]) {
    if (kind == 0)
        hipExtLaunchKernelGGL(la_floor_empty_kernel, dim3((unsigned)nwg), dim3(FLOOR_THREADS), 0, stream, ev[0], ev[1], 0,
                              (int *)out, 0);
    else if (kind == 1)
        launch_stream<FLOOR_FWD_NIN, FLOOR_FWD_NOUT, FLOOR_THREADS>(nwg, in, out, stream, ev);
    else if (kind == 2)
        launch_stream<FLOOR_BWD_NIN, FLOOR_BWD_NOUT, FLOOR_THREADS>(nwg, in, out, stream, ev);
    else if (kind == 3)
        launch_stream<FLOOR_FWD_NIN, FLOOR_FWD_NOUT, FLOOR_SMALL_THREADS>(nwg, in, out, stream, ev);
    else
        launch_stream<FLOOR_BWD_NIN, FLOOR_BWD_NOUT, FLOOR_SMALL_THREADS>(nwg, in, out, stream, ev);
    return hipGetLastError();
}

}  // namespace lachunk
