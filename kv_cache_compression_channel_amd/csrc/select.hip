// select.hip -- H2O cumulative attention scores and recent-window + TopK token selection.
//
// Walkthrough (KV Compression 公式到源码对照) §3.1 (Score(i) = sum over the observed steps of
// a_t(i), an fp32 sum over axis 0 of the [steps][tokens] history), §3.2 (recent window
// [T - W, T) kept, its scores masked to -inf, TopK(B - W) over the rest, sorted unique
// union) and §3.3 (SnapKV: the same selection on one-shot observation scores).
//
// Column sums: each thread owns 4 consecutive tokens and adds the T_obs rows in step
// order (float4 loads, coalesced along tokens), so every score is the same sequence of
// fp32 additions as the definition.
// H2O fused (T <= 32768, T % 4 == 0): one 1024-thread block per row sums the row's history
// straight into registers (8 float4 of scores per thread) and selects from there, so the
// scores never go to memory and back; each block streams its own 4*T_obs*T bytes.
// Selection: one 1024-thread block per row.  Scores become order-preserving 32-bit keys
// (recent tokens lowest, then NaN, then numbers in order, -0 == +0); an MSB-first radix select (8-bit digits over
// the bits where the row's keys differ) finds the k-th largest key t and how many keys
// equal to t are taken (m); a final in-order scan keeps j when key > t, or key == t and
// fewer than m equal keys precede it, or j is recent, and writes kept indices with a
// block prefix sum -- sorted by construction, no sort needed.
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kSumThreads = 256;
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kRegKeys = 32;   // keys per thread kept in registers (T <= 32768)

__global__ void __launch_bounds__(kSumThreads) colsum_kernel(const float* __restrict__ hist, int64_t T_obs,
                                                             int64_t T, float* __restrict__ scores) {
    const int64_t row = blockIdx.y;
    const int64_t j = ((int64_t)blockIdx.x * kSumThreads + threadIdx.x) * 4;
    if (j >= T) return;
    const float* h = hist + row * T_obs * T;
    float* out = scores + row * T;
    if (j + 4 <= T && (T % 4) == 0) {
        float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        int64_t t = 0;
        for (; t + 8 <= T_obs; t += 8) {
            float4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = ld_stream_f4(h + (t + u) * T + j);
#pragma unroll
            for (int u = 0; u < 8; ++u) { acc.x += v[u].x; acc.y += v[u].y; acc.z += v[u].z; acc.w += v[u].w; }
        }
        for (; t < T_obs; ++t) {
            const float4 v = ld_stream_f4(h + t * T + j);
            acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
        }
        *reinterpret_cast<float4*>(out + j) = acc;
    } else {
        for (int64_t c = j; c < j + 4 && c < T; ++c) {
            float acc = 0.0f;
            for (int64_t t = 0; t < T_obs; ++t) acc += h[t * T + c];
            out[c] = acc;
        }
    }
}

__device__ __forceinline__ uint32_t order_key(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 1u;       // NaN: below every number
    if ((u << 1) == 0u) return 0x80000000u;                // -0 and +0 compare equal
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);    // -inf -> 0x007fffff
}
// The recent window's tokens (scores masked to -inf) rank below every earlier token, NaN
// included: for numeric scores this is the -inf mask itself, and it keeps the union of the
// window and the TopK at min(T, max(budget, |window|)) tokens for any scores.
constexpr uint32_t kKeyRecent = 0u;

// Block-wide exclusive prefix of a 0/1 flag; returns the prefix, *total gets the sum.
__device__ __forceinline__ uint32_t block_prefix(bool flag, uint32_t* sh, uint32_t* total) {
    const uint64_t m = __ballot(flag);
    const int lane = threadIdx.x % 64, w = threadIdx.x / 64;
    const uint32_t in_wave = (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
    if (lane == 0) sh[w] = (uint32_t)__popcll(m);
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < kSelWaves; ++i) {
        const uint32_t c = sh[i];
        before += (i < w) ? c : 0u;
        tot += c;
    }
    __syncthreads();
    *total = tot;
    return before + in_wave;
}

template <bool REG>
__global__ void __launch_bounds__(kSelThreads) select_kernel(const float* __restrict__ scores, int64_t T,
                                                             int64_t budget, int64_t window, int64_t K,
                                                             int32_t* __restrict__ keep) {
    __shared__ uint32_t hist[kSelWaves][256];
    __shared__ uint32_t scan[256];
    __shared__ uint32_t sh[kSelWaves];
    __shared__ uint32_t s_min, s_max, s_digit, s_kk;
    const int64_t row = blockIdx.x;
    const float* sc = scores + row * T;
    const int64_t rs = T - window > 0 ? T - window : 0;
    int64_t heavy = budget - (T - rs);
    heavy = heavy < 0 ? 0 : (heavy > T ? T : heavy);
    const int tid = threadIdx.x, w = tid / 64;

    uint32_t kreg[REG ? kRegKeys : 1];
    auto key_at = [&](int64_t j) -> uint32_t { return j >= rs ? kKeyRecent : order_key(sc[j]); };
    if constexpr (REG) {
        // every score loaded (past the end: the last one again), then keyed, so that no load sits
        // behind a per-key branch and waits for the loads before it
        float sv[kRegKeys];
#pragma unroll
        for (int i = 0; i < kRegKeys; ++i) sv[i] = sc[min((int64_t)i * kSelThreads + tid, T - 1)];
#pragma unroll
        for (int i = 0; i < kRegKeys; ++i) {
            const int64_t j = (int64_t)i * kSelThreads + tid;
            kreg[i] = j >= T ? 0u : (j >= rs ? kKeyRecent : order_key(sv[i]));
        }
    }

    // threshold t: the heavy-th largest key; m: how many keys equal to t are taken
    uint32_t thr = 0xffffffffu, take_eq = 0;
    bool none = heavy == 0, all = heavy >= T;
    if (!none && !all) {
        // the bits where this row's keys differ
        uint32_t lo = 0xffffffffu, hi = 0u;
        if constexpr (REG) {
#pragma unroll
            for (int i = 0; i < kRegKeys; ++i)
                if ((int64_t)i * kSelThreads + tid < T) { lo = min(lo, kreg[i]); hi = max(hi, kreg[i]); }
        } else {
            for (int64_t j = tid; j < T; j += kSelThreads) { const uint32_t k = key_at(j); lo = min(lo, k); hi = max(hi, k); }
        }
        for (int off = 32; off >= 1; off /= 2) { lo = min(lo, __shfl_xor(lo, off)); hi = max(hi, __shfl_xor(hi, off)); }
        if (tid == 0) { s_min = 0xffffffffu; s_max = 0u; }
        __syncthreads();
        if (tid % 64 == 0) { atomicMin(&s_min, lo); atomicMax(&s_max, hi); }
        __syncthreads();
        const uint32_t diff = s_min ^ s_max;
        int top = diff ? 31 - __clz((int)diff) : -1;   // highest differing bit
        uint32_t prefix = s_max & (top >= 31 ? 0u : (0xffffffffu << (top + 1)));
        uint32_t pmask = top >= 31 ? 0u : (0xffffffffu << (top + 1));
        uint32_t kk = (uint32_t)heavy;
        while (top >= 0) {
            const int nb = top + 1 >= 8 ? 8 : top + 1;
            const int shift = top + 1 - nb;
            const uint32_t dmask = (1u << nb) - 1u;
            for (int i = tid; i < kSelWaves * 256; i += kSelThreads) (&hist[0][0])[i] = 0u;
            __syncthreads();
            auto count = [&](uint32_t k) {
                if ((k & pmask) == prefix) atomicAdd(&hist[w][(k >> shift) & dmask], 1u);
            };
            if constexpr (REG) {
#pragma unroll
                for (int i = 0; i < kRegKeys; ++i)
                    if ((int64_t)i * kSelThreads + tid < T) count(kreg[i]);
            } else {
                for (int64_t j = tid; j < T; j += kSelThreads) count(key_at(j));
            }
            __syncthreads();
            // digits from the largest down: inclusive running count
            if (tid < 256) {
                uint32_t c = 0;
                const int dgt = 255 - tid;
#pragma unroll
                for (int q = 0; q < kSelWaves; ++q) c += hist[q][dgt];
                scan[tid] = c;
            }
            __syncthreads();
            if (tid < 64) {
                // 256 entries scanned by one wave: 4 per lane, then a wave-wide scan
                uint32_t a0 = scan[4 * tid], a1 = scan[4 * tid + 1], a2 = scan[4 * tid + 2], a3 = scan[4 * tid + 3];
                a1 += a0; a2 += a1; a3 += a2;
                uint32_t run = a3;
                for (int off = 1; off < 64; off *= 2) {
                    const uint32_t o = __shfl_up(run, off);
                    if (tid >= off) run += o;
                }
                const uint32_t base = run - a3;
                const uint32_t inc[4] = {base + a0, base + a1, base + a2, base + a3};
                const uint32_t exc[4] = {base, base + a0, base + a1, base + a2};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (exc[e] < kk && kk <= inc[e]) { s_digit = 255u - (uint32_t)(4 * tid + e); s_kk = kk - exc[e]; }
                }
            }
            __syncthreads();
            prefix |= (s_digit & dmask) << shift;
            pmask |= dmask << shift;
            kk = s_kk;
            top -= nb;
            __syncthreads();
        }
        thr = prefix;
        take_eq = kk;
    }

    // in-order emit
    uint32_t base = 0, eq_seen = 0;
    auto emit = [&](int64_t ch, uint32_t k) {
        const int64_t j = ch * kSelThreads + tid;
        const bool valid = j < T;
        const bool eq = valid && !none && !all && k == thr;
        uint32_t eq_tot;
        const uint32_t eq_rank = eq_seen + block_prefix(eq, sh, &eq_tot);
        const bool take = valid && (all || j >= rs || (!none && (k > thr || (eq && eq_rank < take_eq))));
        uint32_t take_tot;
        const uint32_t pos = base + block_prefix(take, sh, &take_tot);
        if (take && pos < (uint64_t)K) keep[row * K + pos] = (int32_t)j;
        base += take_tot;
        eq_seen += eq_tot;
    };
    const int64_t nchunk = (T + kSelThreads - 1) / kSelThreads;
    if constexpr (REG) {
#pragma unroll
        for (int ch = 0; ch < kRegKeys; ++ch) {
            if (ch >= nchunk) break;
            emit(ch, kreg[ch]);
        }
    } else {
        for (int64_t ch = 0; ch < nchunk; ++ch) {
            const int64_t j = ch * kSelThreads + tid;
            emit(ch, j < T ? key_at(j) : 0u);
        }
    }
}

// Block-wide exclusive prefix of per-thread counts; returns the prefix, *total gets the sum.
__device__ __forceinline__ uint32_t block_prefix_n(uint32_t cnt, uint32_t* sh, uint32_t* total) {
    const int lane = threadIdx.x % 64, w = threadIdx.x / 64;
    uint32_t run = cnt;
#pragma unroll
    for (int off = 1; off < 64; off *= 2) {
        const uint32_t o = __shfl_up(run, off);
        if (lane >= off) run += o;
    }
    if (lane == 63) sh[w] = run;
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < kSelWaves; ++i) {
        const uint32_t c = sh[i];
        before += (i < w) ? c : 0u;
        tot += c;
    }
    __syncthreads();
    *total = tot;
    return before + run - cnt;
}

constexpr int kFusedChunks = 8;   // float4 token groups per thread: 8 x 4 x 1024 = 32768 tokens

// Column sums and selection of one row (Walkthrough §3.1, §3.2).  Thread tid owns tokens
// 4 (i * 1024 + tid) + e, i < 8, e < 4: token order is (i, tid, e) order, which the in-order
// emit follows.  Each score is the same sequence of fp32 additions over the steps as the
// definition.
__global__ void __launch_bounds__(kSelThreads) h2o_fused_kernel(const float* __restrict__ histo, int64_t T_obs,
                                                                int64_t T, int64_t budget, int64_t window, int64_t K,
                                                                float* __restrict__ scores_out,
                                                                int32_t* __restrict__ keep) {
    __shared__ uint32_t hist[kSelWaves][256];
    __shared__ uint32_t scan[256];
    __shared__ uint32_t sh[kSelWaves];
    __shared__ uint32_t s_min, s_max, s_digit, s_kk;
    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x, w = tid / 64;
    const float* hr = histo + row * T_obs * T;
    // T <= 32768 on this path: token indices fit 32 bits
    const int Ti = (int)T;
    const int rs = T - window > 0 ? (int)(T - window) : 0;
    int64_t heavy = budget - (T - rs);
    heavy = heavy < 0 ? 0 : (heavy > T ? T : heavy);

    // ---- column sums: one step's eight float4 loads in flight per thread (read once: streamed) ----
    float4 acc[kFusedChunks];
#pragma unroll
    for (int i = 0; i < kFusedChunks; ++i) acc[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    auto tok = [&](int i) -> int { return 4 * (i * kSelThreads + tid); };
    for (int64_t t = 0; t < T_obs; ++t) {
        float4 a[kFusedChunks];
#pragma unroll
        for (int i = 0; i < kFusedChunks; ++i)
            if (tok(i) < Ti) a[i] = ld_stream_f4(hr + t * T + tok(i));
#pragma unroll
        for (int i = 0; i < kFusedChunks; ++i) {
            if (tok(i) < Ti) { acc[i].x += a[i].x; acc[i].y += a[i].y; acc[i].z += a[i].z; acc[i].w += a[i].w; }
        }
    }
    if (scores_out) {
#pragma unroll
        for (int i = 0; i < kFusedChunks; ++i)
            if (tok(i) < Ti) *reinterpret_cast<float4*>(scores_out + row * T + tok(i)) = acc[i];
    }
    if (K == 0) return;

    // ---- keys: order-preserving, recent tokens lowest, past the end 0 (never counted) ----
    uint32_t kreg[kFusedChunks][4];
#pragma unroll
    for (int i = 0; i < kFusedChunks; ++i) {
        const float v[4] = {acc[i].x, acc[i].y, acc[i].z, acc[i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int j = tok(i) + e;
            kreg[i][e] = j >= Ti ? 0u : (j >= rs ? kKeyRecent : order_key(v[e]));
        }
    }

    // ---- threshold t: the heavy-th largest key; m: how many keys equal to t are taken ----
    uint32_t thr = 0xffffffffu, take_eq = 0;
    const bool none = heavy == 0, all = heavy >= T;
    if (!none && !all) {
        uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
        for (int i = 0; i < kFusedChunks; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (tok(i) + e < Ti) { lo = min(lo, kreg[i][e]); hi = max(hi, kreg[i][e]); }
        for (int off = 32; off >= 1; off /= 2) { lo = min(lo, __shfl_xor(lo, off)); hi = max(hi, __shfl_xor(hi, off)); }
        if (tid == 0) { s_min = 0xffffffffu; s_max = 0u; }
        __syncthreads();
        if (tid % 64 == 0) { atomicMin(&s_min, lo); atomicMax(&s_max, hi); }
        __syncthreads();
        const uint32_t diff = s_min ^ s_max;
        int top = diff ? 31 - __clz((int)diff) : -1;   // highest differing bit
        uint32_t prefix = s_max & (top >= 31 ? 0u : (0xffffffffu << (top + 1)));
        uint32_t pmask = top >= 31 ? 0u : (0xffffffffu << (top + 1));
        uint32_t kk = (uint32_t)heavy;
        while (top >= 0) {
            const int nb = top + 1 >= 8 ? 8 : top + 1;
            const int shift = top + 1 - nb;
            const uint32_t dmask = (1u << nb) - 1u;
            for (int q = tid; q < kSelWaves * 256; q += kSelThreads) (&hist[0][0])[q] = 0u;
            __syncthreads();
#pragma unroll
            for (int i = 0; i < kFusedChunks; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t k = kreg[i][e];
                    if (tok(i) + e < Ti && (k & pmask) == prefix) atomicAdd(&hist[w][(k >> shift) & dmask], 1u);
                }
            __syncthreads();
            // digits from the largest down: inclusive running count
            if (tid < 256) {
                uint32_t c = 0;
                const int dgt = 255 - tid;
#pragma unroll
                for (int q = 0; q < kSelWaves; ++q) c += hist[q][dgt];
                scan[tid] = c;
            }
            __syncthreads();
            if (tid < 64) {
                uint32_t a0 = scan[4 * tid], a1 = scan[4 * tid + 1], a2 = scan[4 * tid + 2], a3 = scan[4 * tid + 3];
                a1 += a0; a2 += a1; a3 += a2;
                uint32_t run = a3;
                for (int off = 1; off < 64; off *= 2) {
                    const uint32_t o = __shfl_up(run, off);
                    if (tid >= off) run += o;
                }
                const uint32_t base = run - a3;
                const uint32_t inc[4] = {base + a0, base + a1, base + a2, base + a3};
                const uint32_t exc[4] = {base, base + a0, base + a1, base + a2};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (exc[e] < kk && kk <= inc[e]) { s_digit = 255u - (uint32_t)(4 * tid + e); s_kk = kk - exc[e]; }
                }
            }
            __syncthreads();
            prefix |= (s_digit & dmask) << shift;
            pmask |= dmask << shift;
            kk = s_kk;
            top -= nb;
            __syncthreads();
        }
        thr = prefix;
        take_eq = kk;
    }

    // ---- in-order emit: chunk i, then thread, then e ----
    uint32_t base = 0, eq_seen = 0;
#pragma unroll
    for (int i = 0; i < kFusedChunks; ++i) {
        if (i * kSelThreads * 4 >= Ti) break;
        bool eq[4];
        uint32_t neq = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            eq[e] = tok(i) + e < Ti && !none && !all && kreg[i][e] == thr;
            neq += eq[e] ? 1u : 0u;
        }
        uint32_t eq_tot;
        uint32_t eq_rank = eq_seen + block_prefix_n(neq, sh, &eq_tot);
        bool take[4];
        uint32_t ntake = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int j = tok(i) + e;
            const uint32_t k = kreg[i][e];
            take[e] = j < Ti && (all || j >= rs || (!none && (k > thr || (eq[e] && eq_rank < take_eq))));
            if (eq[e]) ++eq_rank;
            ntake += take[e] ? 1u : 0u;
        }
        uint32_t take_tot;
        uint32_t pos = base + block_prefix_n(ntake, sh, &take_tot);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (take[e]) {
                if (pos < (uint64_t)K) keep[row * K + pos] = (int32_t)(tok(i) + e);
                ++pos;
            }
        }
        base += take_tot;
        eq_seen += eq_tot;
    }
}

int select_launch(const float* scores, int64_t rows, int64_t T, int64_t budget, int64_t window, int32_t* keep,
                  hipStream_t st) {
    const int64_t K = kvq_keep_count(T, budget, window);
    if (T <= (int64_t)kRegKeys * kSelThreads)
        hipLaunchKernelGGL((select_kernel<true>), dim3((unsigned)rows), dim3(kSelThreads), 0, st, scores, T, budget,
                           window, K, keep);
    else
        hipLaunchKernelGGL((select_kernel<false>), dim3((unsigned)rows), dim3(kSelThreads), 0, st, scores, T, budget,
                           window, K, keep);
    return launch_status("token selection");
}

}  // namespace
}  // namespace kvq

extern "C" {

size_t kvq_select_ws(int64_t rows, int64_t T) {
    if (rows < 1 || T < 1) return 0;
    return (size_t)(rows * T) * sizeof(float);
}

int kvq_h2o_select(const float* hist, int64_t rows, int64_t T_obs, int64_t T, int64_t budget, int64_t window,
                   float* scores_or_null, int32_t* keep, void* ws, size_t ws_bytes, kvq_stream stream) {
    const int64_t K = kvq_keep_count(T, budget, window);
    KVQ_REQUIRE(hist && (keep || K == 0), "kvq_h2o_select: NULL hist or keep");
    KVQ_REQUIRE(rows >= 1 && T_obs >= 1 && T >= 1, "kvq_h2o_select: rows, T_obs, T must be >= 1");
    KVQ_REQUIRE(T <= 0x7fffffff && rows <= 0x7fffffff, "kvq_h2o_select: T and rows must fit int32");
    KVQ_REQUIRE(budget >= 0 && window >= 0, "kvq_h2o_select: budget and window must be >= 0");
    KVQ_REQUIRE(rows <= 65535, "kvq_h2o_select: rows must be <= 65535");
    float* scores = scores_or_null;
    if (!scores) {
        KVQ_REQUIRE(ws && ws_bytes >= kvq_select_ws(rows, T), "kvq_h2o_select: workspace of %zu bytes needed",
                    kvq_select_ws(rows, T));
        scores = static_cast<float*>(ws);
    }
    KVQ_REQUIRE_ALIGNED(hist, "hist");
    KVQ_REQUIRE_ALIGNED(scores, "scores");
    KVQ_REQUIRE_ALIGNED(keep, "keep");
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (K > 0 && T % 4 == 0 && T <= (int64_t)kvq::kFusedChunks * 4 * kvq::kSelThreads) {
        hipLaunchKernelGGL(kvq::h2o_fused_kernel, dim3((unsigned)rows), dim3(kvq::kSelThreads), 0, st, hist, T_obs, T,
                           budget, window, K, scores_or_null, keep);
        return kvq::launch_status("H2O selection");
    }
    const dim3 grid((unsigned)kvq::cdiv(kvq::cdiv(T, 4), kvq::kSumThreads), (unsigned)rows);
    hipLaunchKernelGGL(kvq::colsum_kernel, grid, dim3(kvq::kSumThreads), 0, st, hist, T_obs, T, scores);
    const int rc = kvq::launch_status("H2O column sums");
    if (rc || K == 0) return rc;   // nothing to keep: only the scores are produced
    return kvq::select_launch(scores, rows, T, budget, window, keep, st);
}

int kvq_snapkv_select(const float* scores, int64_t rows, int64_t T, int64_t budget, int64_t window, int32_t* keep,
                      void* ws, size_t ws_bytes, kvq_stream stream) {
    (void)ws;
    (void)ws_bytes;
    const int64_t K = kvq_keep_count(T, budget, window);
    KVQ_REQUIRE(scores && (keep || K == 0), "kvq_snapkv_select: NULL scores or keep");
    KVQ_REQUIRE(rows >= 1 && T >= 1, "kvq_snapkv_select: rows, T must be >= 1");
    KVQ_REQUIRE(T <= 0x7fffffff && rows <= 0x7fffffff, "kvq_snapkv_select: T and rows must fit int32");
    KVQ_REQUIRE(budget >= 0 && window >= 0, "kvq_snapkv_select: budget and window must be >= 0");
    KVQ_REQUIRE_ALIGNED(scores, "scores");
    KVQ_REQUIRE_ALIGNED(keep, "keep");
    if (K == 0) return KVQ_OK;
    return kvq::select_launch(scores, rows, T, budget, window, keep, static_cast<hipStream_t>(stream));
}

}  // extern "C"
