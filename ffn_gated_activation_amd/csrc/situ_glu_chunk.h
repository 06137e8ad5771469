// The chunk layout of the 128-bit elementwise kernels, shared by the bf16 /
// fp32 kernels and the MXFP8 forward: a row is cut into chunks of 64 lanes x
// one 16-byte vector of each input stream (1 KiB of each half row); a
// wavefront takes k consecutive chunks of the row-major chunk numbering and
// issues the next chunk's loads before the current chunk's math.  Included by
// the .hip sources only.
#pragma once

#include "situ_glu_device.h"

namespace situ {
namespace {

constexpr uint32_t kChunkBytes = 1024;  // 64 lanes x 16 bytes of each stream

// One chunk's streams: buffer descriptors (range = the chunk, or empty for a
// chunk past the wavefront's share: loads return zeros, stores are dropped)
// and the bits of the row's routing weight (fp32, or bf16 in the low half),
// converted only by the chunk's math.  The weight's dtype is a template
// parameter (RWB: bf16), so that no chunk's loads wait behind a branch on it
// or behind the weight's own load.
template <int NIN, int NOUT>
struct Chunk {
    rsrc_t in[NIN];
    rsrc_t out[NOUT];
    uint32_t rbits;
};

template <bool RWB>
__device__ __forceinline__ float weight_of(uint32_t rbits)
{
    return __uint_as_float(RWB ? rbits << 16 : rbits);
}

// Bits of routing weight i (fp32, or bf16 in the low half).
template <bool RWB>
__device__ __forceinline__ uint32_t weight_bits(const void *rw, int64_t i)
{
    return RWB ? (uint32_t)static_cast<const uint16_t *>(rw)[i] : static_cast<const uint32_t *>(rw)[i];
}

// Fences that keep each chunk's loads ahead of the previous chunk's math, as
// written: the scheduling barrier within a block, and an empty statement
// that may touch memory, so that no load is sunk past a branch of the math
// (it emits no instruction).
__device__ __forceinline__ void order_fence()
{
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
}

// Issue one chunk's loads.
template <int NIN, int NOUT>
__device__ __forceinline__ void load_chunk(uint4 *v, const Chunk<NIN, NOUT> &k, uint32_t voff)
{
#pragma unroll
    for (int i = 0; i < NIN; ++i)
        v[i] = bload(k.in[i], voff);
    order_fence();
}

// chunk index -> (row, chunk in row)
__device__ __forceinline__ void locate(uint32_t u, const ChunkGeom &g, int64_t &row, uint32_t &c)
{
    const uint32_t q = g.cpr == 1 ? u : __umulhi(u, g.magic) >> g.shift;
    row = q;
    c = u - q * (uint32_t)g.cpr;
}

// The wavefront's n chunks (n >= 1), two register sets: the loads of chunk
// i + 1 are in flight during chunk i's math.  `step(row, c)` moves to the
// next chunk.  MAKE(row, c, live) builds a chunk's descriptors; BODY(regs,
// chunk) is the math and the stores.
#define SITU_CHUNK_PIPELINE(NIN, NOUT, MAKE, BODY)                                                       \
    {                                                                                             \
        uint4 A[NIN], B[NIN];                                                                     \
        Chunk<NIN, NOUT> ka = MAKE(row, c, true); \
        load_chunk(A, ka, voff);                                                                  \
        step(row, c);                                                                             \
        Chunk<NIN, NOUT> kb = MAKE(row, c, 1 < n); \
        load_chunk(B, kb, voff);                                                                  \
        BODY(A, ka);                                                                              \
        int i = 1;                                                                                \
        for (; i + 2 <= n; i += 2) {                                                              \
            step(row, c);                                                                         \
            ka = MAKE(row, c, i + 1 < n);  \
            load_chunk(A, ka, voff);                                                              \
            BODY(B, kb);                                                                          \
            step(row, c);                                                                         \
            kb = MAKE(row, c, i + 2 < n);  \
            load_chunk(B, kb, voff);                                                              \
            BODY(A, ka);                                                                          \
        }                                                                                         \
        if (i < n) {                                                                              \
            BODY(B, kb);                                                                          \
        }                                                                                         \
    }

}  // namespace
}  // namespace situ
