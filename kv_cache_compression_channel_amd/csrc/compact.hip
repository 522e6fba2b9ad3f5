// compact.hip -- eviction as compaction: gather the kept KV rows of every (b, h) into a
// dense cache (Explainer (KV cache 压缩：把历史装得更小), eviction section: only the
// selected KV are kept; later queries read only what was kept).
//
// dst[b][k][h][:] = src[b][keep[b][h][k]][h][:].  One thread moves 16 bytes; d/8 threads
// move one 2d-byte row, so reads and writes are whole 128-byte lines for d >= 64.  A keep
// entry outside [0, T) is clamped into range (two integer operations), so a bad index
// yields an unspecified row, never an access outside the source.
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;

__global__ void __launch_bounds__(kThreads) compact_kernel(const uint16_t* __restrict__ ks,
                                                           const uint16_t* __restrict__ vs, int64_t T, int64_t H,
                                                           int64_t d, const int32_t* __restrict__ keep, int64_t K,
                                                           int64_t nrows, uint16_t* __restrict__ kd,
                                                           uint16_t* __restrict__ vd) {
    // chunk and row counts fit 31 bits (the host checks): index arithmetic in 32 bits
    const uint32_t cpr = (uint32_t)(d / 8);   // 16-byte chunks per row
    const uint32_t total = (uint32_t)(nrows * cpr);
    const uint32_t Hu = (uint32_t)H, Ku = (uint32_t)K;
    for (uint32_t i = blockIdx.x * kThreads + threadIdx.x; i < total; i += gridDim.x * kThreads) {
        const uint32_t row = i / cpr, c = i - row * cpr;
        // destination row order [b][k][h]
        const uint32_t q = row / Hu;
        const int64_t h = row - q * Hu, k = q % Ku, b = q / Ku;
        const int32_t tk = keep[(b * H + h) * K + k];
        const int64_t t = tk < 0 ? 0 : (tk >= T ? T - 1 : (int64_t)tk);
        const int64_t so = ((b * T + t) * H + h) * d + 8 * c;
        const int64_t dof = row * d + 8 * c;
        *reinterpret_cast<uint4*>(kd + dof) = *reinterpret_cast<const uint4*>(ks + so);
        if (vs) *reinterpret_cast<uint4*>(vd + dof) = *reinterpret_cast<const uint4*>(vs + so);
    }
}

}  // namespace
}  // namespace kvq

extern "C" int kvq_compact(const void* k_src, const void* v_src_or_null, int64_t B, int64_t T, int64_t H, int64_t d,
                           const int32_t* keep, int64_t K, void* k_dst, void* v_dst_or_null, kvq_stream stream) {
    KVQ_REQUIRE(k_src && k_dst && keep, "kvq_compact: NULL k_src, k_dst or keep");
    KVQ_REQUIRE((v_src_or_null == nullptr) == (v_dst_or_null == nullptr),
                "kvq_compact: give both v_src and v_dst or neither");
    KVQ_REQUIRE(B >= 1 && T >= 1 && H >= 1 && d >= 1 && K >= 1, "kvq_compact: B, T, H, d, K must be >= 1");
    KVQ_REQUIRE(K <= T, "kvq_compact: K (%lld) > T (%lld)", (long long)K, (long long)T);
    KVQ_REQUIRE(d % 8 == 0, "kvq_compact: d must be a multiple of 8");
    KVQ_REQUIRE(B * T * H * d < ((int64_t)1 << 40), "kvq_compact: cache too large");
    KVQ_REQUIRE_ALIGNED(k_src, "k_src");
    KVQ_REQUIRE_ALIGNED(k_dst, "k_dst");
    KVQ_REQUIRE_ALIGNED(v_src_or_null, "v_src");
    KVQ_REQUIRE_ALIGNED(v_dst_or_null, "v_dst");
    KVQ_REQUIRE_ALIGNED(keep, "keep");
    const int64_t nrows = B * K * H;
    const int64_t total = nrows * (d / 8);
    KVQ_REQUIRE(total < ((int64_t)1 << 31), "kvq_compact: more than 2^31 16-byte chunks to move");
    const unsigned blocks = (unsigned)std::min<int64_t>(kvq::cdiv(total, kvq::kThreads), 1 << 16);
    hipLaunchKernelGGL(kvq::compact_kernel, dim3(blocks), dim3(kvq::kThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint16_t*>(k_src), static_cast<const uint16_t*>(v_src_or_null), T, H, d, keep,
                       K, nrows, static_cast<uint16_t*>(k_dst), static_cast<uint16_t*>(v_dst_or_null));
    return kvq::launch_status("kvq_compact");
}
