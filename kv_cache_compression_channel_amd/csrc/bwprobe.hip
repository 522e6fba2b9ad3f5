// bwprobe.hip -- streaming bandwidth probes: what this device sustains for a read-only, a
// write-only and a read+write stream in a given byte ratio, with the same 16-byte loads and
// stores (plain or non-temporal) the kernels of this library use.  A kernel's time is then
// read against the probe of its own read:write mix as well as against the nominal HBM peak.
//
// One kernel shape for every mix, shaped like the library's streaming kernels: each
// workgroup moves one tile and exits -- every thread issues its A loads (each instruction a
// contiguous 4 KiB per workgroup), then B stores of a value that depends on them (as a
// quantizer's output depends on its input), so no load can be dropped.  The depth scales A and
// B together: on MI355X short tiles (one or two accesses per thread) stream stores markedly
// faster than eight (6.8 against 5.7 TB/s write-only), so a ceiling is the best over depths.
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kBwThreads = 256;

template <int A, int B, bool NT>
__global__ void __launch_bounds__(kBwThreads) bw_kernel(const uint4* __restrict__ src, int64_t r16,
                                                        uint4* __restrict__ dst, int64_t w16) {
    const int64_t u = blockIdx.x;
    const int t = threadIdx.x;
    uint32_t acc = (uint32_t)t;
    if constexpr (A > 0) {
        uint4 v[A];
#pragma unroll
        for (int i = 0; i < A; ++i) {
            const int64_t idx = (u * A + i) * kBwThreads + t;
            if (idx < r16) v[i] = NT ? ld_stream_u4(src + idx) : src[idx];
        }
#pragma unroll
        for (int i = 0; i < A; ++i) {
            const int64_t idx = (u * A + i) * kBwThreads + t;
            if (idx < r16) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
        }
    }
    if constexpr (B > 0) {
#pragma unroll
        for (int i = 0; i < B; ++i) {
            const int64_t idx = (u * B + i) * kBwThreads + t;
            const uint4 o = make_uint4(acc ^ (uint32_t)i, acc, acc, acc);
            if (idx < w16) {
                if constexpr (NT) st_stream_u4(dst + idx, o);
                else dst[idx] = o;
            }
        }
    }
    // a read-only stream keeps its loads live through a store that (almost) never happens
    if constexpr (B == 0) {
        if (acc == 0x9e3779b9u) dst[0] = make_uint4(acc, acc, acc, acc);
    }
}

template <int A, int B, bool NT>
void launch_bw(const void* src, int64_t r16, void* dst, int64_t w16, hipStream_t st) {
    int64_t blocks = 0;
    if (A > 0) blocks = std::max<int64_t>(blocks, cdiv(r16, (int64_t)A * kBwThreads));
    if (B > 0) blocks = std::max<int64_t>(blocks, cdiv(w16, (int64_t)B * kBwThreads));
    hipLaunchKernelGGL((bw_kernel<A, B, NT>), dim3((unsigned)blocks), dim3(kBwThreads), 0, st,
                       static_cast<const uint4*>(src), r16, static_cast<uint4*>(dst), w16);
}

template <int A, int B>
void launch_bw_nt(const void* src, int64_t r16, void* dst, int64_t w16, int nt, hipStream_t st) {
    if (nt) launch_bw<A, B, true>(src, r16, dst, w16, st);
    else launch_bw<A, B, false>(src, r16, dst, w16, st);
}

// the base pattern (A, B) times depth 1, 2, 4 or 8
template <int A, int B>
void launch_bw_depth(const void* src, int64_t r16, void* dst, int64_t w16, int nt, int depth, hipStream_t st) {
    switch (depth) {
        case 1: launch_bw_nt<A, B>(src, r16, dst, w16, nt, st); break;
        case 2: launch_bw_nt<2 * A, 2 * B>(src, r16, dst, w16, nt, st); break;
        case 4: launch_bw_nt<4 * A, 4 * B>(src, r16, dst, w16, nt, st); break;
        default: launch_bw_nt<8 * A, 8 * B>(src, r16, dst, w16, nt, st); break;
    }
}

}  // namespace
}  // namespace kvq

extern "C" int kvq_bw_probe(const void* src, uint64_t read_bytes, void* dst, uint64_t write_bytes, int nt, int depth,
                            kvq_stream stream) {
    KVQ_REQUIRE(dst, "kvq_bw_probe: NULL dst (a read-only probe needs a 16-byte sink)");
    KVQ_REQUIRE(read_bytes == 0 || src, "kvq_bw_probe: NULL src");
    KVQ_REQUIRE(read_bytes % 16 == 0 && write_bytes % 16 == 0, "kvq_bw_probe: sizes must be multiples of 16");
    KVQ_REQUIRE(read_bytes + write_bytes > 0, "kvq_bw_probe: nothing to move");
    // the grid (one workgroup per 4 KiB x the larger part of the mix) must fit 32 bits
    KVQ_REQUIRE(read_bytes < ((uint64_t)1 << 42) && write_bytes < ((uint64_t)1 << 42), "kvq_bw_probe: too large");
    KVQ_REQUIRE(depth == 1 || depth == 2 || depth == 4 || depth == 8, "kvq_bw_probe: depth must be 1, 2, 4 or 8");
    KVQ_REQUIRE_ALIGNED(src, "src");
    KVQ_REQUIRE_ALIGNED(dst, "dst");
    const int64_t r16 = (int64_t)(read_bytes / 16), w16 = (int64_t)(write_bytes / 16);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const uint64_t r = read_bytes, w = write_bytes;
    if (w == 0) kvq::launch_bw_depth<1, 0>(src, r16, dst, w16, nt, depth, st);
    else if (r == 0) kvq::launch_bw_depth<0, 1>(src, r16, dst, w16, nt, depth, st);
    else if (r == w) kvq::launch_bw_depth<1, 1>(src, r16, dst, w16, nt, depth, st);
    else if (r == 2 * w) kvq::launch_bw_depth<2, 1>(src, r16, dst, w16, nt, depth, st);
    else if (2 * r == w) kvq::launch_bw_depth<1, 2>(src, r16, dst, w16, nt, depth, st);
    else if (9 * r == 32 * w || 32 * r == 9 * w) {
        KVQ_REQUIRE(depth == 1, "kvq_bw_probe: the 32:9 and 9:32 mixes take depth 1 (32 + 9 accesses per thread)");
        if (9 * r == 32 * w) kvq::launch_bw_nt<32, 9>(src, r16, dst, w16, nt, st);
        else kvq::launch_bw_nt<9, 32>(src, r16, dst, w16, nt, st);
    } else {
        return kvq::fail(KVQ_EINVAL, "kvq_bw_probe: read:write must be 1:0, 0:1, 1:1, 2:1, 1:2, 32:9 or 9:32");
    }
    return kvq::launch_status("kvq_bw_probe");
}
