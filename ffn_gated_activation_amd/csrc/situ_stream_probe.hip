// Bandwidth probe for the benchmark: a plain streaming kernel with the
// SiTU-GLU kernels' access pattern and no arithmetic, for a given mix of
// read and written streams.  Not part of the SiTU-GLU library or its
// boundary; built as its own shared library (libsitu_stream_probe.so) and
// used only to report the memory ceiling of each read:write mix next to
// the measured kernels.
//
// Access pattern, as one chunk of the 128-bit path of the forward and
// backward: one 64-lane wavefront per workgroup, each wavefront one chunk of
// 64 lanes x one 16-byte vector of every stream (1 KiB per stream), the
// loads issued before the stores, every access through a buffer descriptor
// with the non-temporal hint.  The written value is the xor of the read
// vectors, so no load can be dropped.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
using rsrc_t = __amdgpu_buffer_rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format
constexpr int kStreaming = 2;           // cache policy operand: nt
constexpr int kMaxIn = 4, kMaxOut = 2;

struct Streams {
    const char *in[kMaxIn];
    char *out[kMaxOut];
};

__device__ __forceinline__ rsrc_t rsrc(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, kRsrcWord3);
}

template <int NI, int NO>
__global__ void __launch_bounds__(64) situ_stream_probe_kernel(Streams s, int64_t nvec)
{
    constexpr int kUnroll = 1;
    constexpr int kStripVecs = 64 * kUnroll;
    const int lane = threadIdx.x;
    const int64_t v0 = (int64_t)blockIdx.x * kStripVecs;
    const int64_t left = nvec - v0;
    const uint32_t bytes = (uint32_t)(left < kStripVecs ? left : kStripVecs) * 16u;
    u32x4 x[NI][kUnroll];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const rsrc_t r = rsrc(s.in[i] + v0 * 16, bytes);
#pragma unroll
        for (int k = 0; k < kUnroll; ++k)
            x[i][k] = __builtin_amdgcn_raw_buffer_load_b128(r, (int)((64 * k + lane) * 16), 0, kStreaming);
    }
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
        u32x4 v = x[0][k];
#pragma unroll
        for (int i = 1; i < NI; ++i)
            v ^= x[i][k];
#pragma unroll
        for (int o = 0; o < NO; ++o)
            __builtin_amdgcn_raw_buffer_store_b128(v + (unsigned)o, rsrc(s.out[o] + v0 * 16, bytes),
                                                   (int)((64 * k + lane) * 16), 0, kStreaming);
    }
}

template <int NI, int NO>
hipError_t launch(const Streams &s, int64_t nvec, hipStream_t st)
{
    constexpr int kStripVecs = 64;
    const int64_t blocks = (nvec + kStripVecs - 1) / kStripVecs;
    hipLaunchKernelGGL((situ_stream_probe_kernel<NI, NO>), dim3((unsigned)blocks), dim3(64), 0, st, s, nvec);
    return hipGetLastError();
}

}  // namespace

// Reads n_in streams and writes n_out streams of `bytes` bytes each
// (device pointers, 16-byte aligned; bytes a multiple of 16 and at most
// 2^40); output o receives the xor of the inputs plus o.  Enqueued on
// `stream` (a hipStream_t; NULL = the default stream).  Returns 0, or 1 for
// an invalid argument (nothing is launched), or 3 for a launch error.
extern "C" int situ_stream_probe(const void *const *in, int n_in, void *const *out, int n_out, int64_t bytes,
                                 void *stream)
{
    if (!in || !out || n_in < 1 || n_in > kMaxIn || n_out < 1 || n_out > kMaxOut || bytes < 0 || bytes % 16 ||
        bytes > ((int64_t)1 << 40))
        return 1;
    Streams s = {};
    for (int i = 0; i < n_in; ++i) {
        if (!in[i] || (uintptr_t)in[i] % 16)
            return 1;
        s.in[i] = static_cast<const char *>(in[i]);
    }
    for (int o = 0; o < n_out; ++o) {
        if (!out[o] || (uintptr_t)out[o] % 16)
            return 1;
        s.out[o] = static_cast<char *>(out[o]);
    }
    const int64_t nvec = bytes / 16;
    if (nvec == 0)
        return 0;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t err = hipErrorInvalidValue;
    switch (n_in * 10 + n_out) {
    case 11: err = launch<1, 1>(s, nvec, st); break;
    case 12: err = launch<1, 2>(s, nvec, st); break;
    case 21: err = launch<2, 1>(s, nvec, st); break;
    case 22: err = launch<2, 2>(s, nvec, st); break;
    case 31: err = launch<3, 1>(s, nvec, st); break;
    case 32: err = launch<3, 2>(s, nvec, st); break;
    case 41: err = launch<4, 1>(s, nvec, st); break;
    case 42: err = launch<4, 2>(s, nvec, st); break;
    default: return 1;
    }
    return err == hipSuccess ? 0 : 3;
}
