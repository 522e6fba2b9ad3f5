// mixed.hip -- per-token mixed precision: every row (token) is stored at 2, 4, 8 or 16 bits as its
// 2-bit tag says, rows of one width together in that width's pool.
//
// Adaptive-bit blog (自适应量化框架): §2.1 four precision levels 2/4/8/16 chosen per token by a
// controller (the controller is not part of this library: tags are inputs); §3.1 per-token
// dynamic quantization, symmetric at 2 and 4 bits, asymmetric at 8 bits; §3.2 2-bit precision
// tags (00/01/10/11 = 2/4/8/16 bits) and tokens of one precision stored contiguously.  The
// symmetric and asymmetric steps are those of the Walkthrough (KV Compression 公式到源码对照)
// §1.1 and §1.2, taken over a row instead of over a channel.
//
// kvq_mixed_plan: slot[r] = number of earlier rows with the tag of row r (the row's place in its
//   pool) and the four pool sizes.  Three launches: per-block tag counts (1024 rows per block,
//   four rows = one tag byte per thread), a scan of the block counts, then per-row ranks inside the
//   block.  The four counters travel packed in 16-bit fields of one 64-bit word, so a single block
//   scan serves all four tags.
// kvq_mixed_quant / kvq_mixed_dequant: C/8 lanes per row (at most 64), 8 channels per lane and
//   chunk; the row's reduction (absmax, or min and max) finishes with xor shuffles inside the
//   row's lanes.
#include "int4_common.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;
constexpr int kPlanRows = 1024;   // rows per plan block (one tag byte per thread)

__device__ __forceinline__ int tag_at(uint32_t byte, int i) { return (int)((byte >> (2 * i)) & 3u); }

// The store descriptor in scalar registers.  It arrives in kernel-argument memory, where a
// per-lane index (the capacity of a row's tag) or a per-lane choice between two of its pointers
// (the scale array of a 2- or 4-bit row) compiles to a load from that memory, and then a load
// through the pointer it returns, in front of every pool access: two dependent round trips per
// row.  Values passed through readfirstlane are plain registers to the compiler.
__device__ __forceinline__ uint32_t sgpr32(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t sgpr64(int64_t v) {
    const uint64_t u = (uint64_t)v;
    return (int64_t)(((uint64_t)sgpr32((uint32_t)(u >> 32)) << 32) | sgpr32((uint32_t)u));
}
// (through a global-address-space pointer, so accesses stay global loads and stores)
template <typename T>
__device__ __forceinline__ T* sgprp(T* p) {
    typedef __attribute__((address_space(1))) T gT;
    return (T*)(gT*)(uintptr_t)sgpr64(reinterpret_cast<int64_t>(p));
}
__device__ __forceinline__ kvq_mixed_store store_in_sregs(const kvq_mixed_store& a) {
    kvq_mixed_store m;
    m.N = sgpr64(a.N);
    m.C = sgpr64(a.C);
    m.tags = sgprp(a.tags);
    m.slot = sgprp(a.slot);
#pragma unroll
    for (int i = 0; i < 4; ++i) m.cap[i] = sgpr64(a.cap[i]);
    m.q2 = sgprp(a.q2);
    m.s2 = sgprp(a.s2);
    m.q4 = sgprp(a.q4);
    m.s4 = sgprp(a.s4);
    m.q8 = sgprp(a.q8);
    m.s8 = sgprp(a.s8);
    m.z8 = sgprp(a.z8);
    m.x16 = sgprp(a.x16);
    return m;
}
// Capacity of tag t's pool, selected among the four values.
__device__ __forceinline__ int64_t cap_of(const kvq_mixed_store& m, int t) {
    return t == 0 ? m.cap[0] : t == 1 ? m.cap[1] : t == 2 ? m.cap[2] : m.cap[3];
}

// Inclusive scan over the block of a 64-bit word of four 16-bit counters (sums stay below 2^16).
__device__ __forceinline__ uint64_t block_scan_u64(uint64_t v, uint64_t* s_w) {
    const int tid = threadIdx.x, lane = tid % 64, w = tid / 64;
#pragma unroll
    for (int off = 1; off < 64; off *= 2) {
        const uint64_t o = __shfl_up(v, off);
        if (lane >= off) v += o;
    }
    if (lane == 63) s_w[w] = v;
    __syncthreads();
    uint64_t base = 0;
    for (int i = 0; i < w; ++i) base += s_w[i];
    return v + base;
}

__global__ void __launch_bounds__(kThreads) mixed_count_kernel(const uint8_t* __restrict__ tags, int64_t N,
                                                              uint64_t* __restrict__ blk) {
    __shared__ uint64_t s_w[kThreads / 64];
    const int64_t r0 = (int64_t)blockIdx.x * kPlanRows + 4 * threadIdx.x;
    uint64_t c = 0;
    if (r0 < N) {
        const uint32_t byte = tags[r0 / 4];
        for (int i = 0; i < 4 && r0 + i < N; ++i) c += (uint64_t)1 << (16 * tag_at(byte, i));
    }
    const uint64_t inc = block_scan_u64(c, s_w);
    if (threadIdx.x == kThreads - 1) blk[blockIdx.x] = inc;
}

// One block: exclusive prefix of the block counts (in place, as 4 x 32-bit offsets per block) and
// the totals.  Offsets can pass 2^16, so they are widened to 32-bit fields here.
__global__ void __launch_bounds__(1024) mixed_scan_kernel(uint64_t* __restrict__ blk, uint4* __restrict__ off,
                                                         int64_t nblk, int64_t* __restrict__ counts) {
    __shared__ uint32_t s_part[1024 / 64][4];
    const int tid = threadIdx.x, lane = tid % 64, w = tid / 64;
    uint32_t carry[4] = {0u, 0u, 0u, 0u};
    for (int64_t b0 = 0; b0 < nblk; b0 += 1024) {
        const int64_t b = b0 + tid;
        const uint64_t v = b < nblk ? blk[b] : 0;
        uint32_t x[4], inc[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            x[k] = (uint32_t)((v >> (16 * k)) & 0xffffu);
            inc[k] = x[k];
        }
#pragma unroll
        for (int d = 1; d < 64; d *= 2) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t o = __shfl_up(inc[k], d);
                if (lane >= d) inc[k] += o;
            }
        }
        if (lane == 63) {
#pragma unroll
            for (int k = 0; k < 4; ++k) s_part[w][k] = inc[k];
        }
        __syncthreads();
        uint32_t base[4] = {carry[0], carry[1], carry[2], carry[3]};
        for (int i = 0; i < w; ++i) {
#pragma unroll
            for (int k = 0; k < 4; ++k) base[k] += s_part[i][k];
        }
        if (b < nblk) off[b] = make_uint4(base[0] + inc[0] - x[0], base[1] + inc[1] - x[1], base[2] + inc[2] - x[2],
                                          base[3] + inc[3] - x[3]);
        uint32_t tot[4] = {0u, 0u, 0u, 0u};
        for (int i = 0; i < 1024 / 64; ++i) {
#pragma unroll
            for (int k = 0; k < 4; ++k) tot[k] += s_part[i][k];
        }
        __syncthreads();   // s_part is rewritten by the next chunk
#pragma unroll
        for (int k = 0; k < 4; ++k) carry[k] += tot[k];
    }
    if (tid == 0) {
#pragma unroll
        for (int k = 0; k < 4; ++k) counts[k] = carry[k];
    }
}

// Slots of one block's rows.  off != NULL: the block's offset in each pool comes from the scan
// kernel.  off == NULL (at most kSelfPrefixBlocks blocks): every block sums the count words of the
// blocks before it itself (at most that many 8-byte words, from L2), which saves the scan launch
// between the count and slot passes; block 0 sums all of them and writes the totals.
constexpr int64_t kSelfPrefixBlocks = 4096;
__global__ void __launch_bounds__(kThreads) mixed_slot_kernel(const uint8_t* __restrict__ tags, int64_t N,
                                                             const uint4* __restrict__ off,
                                                             const uint64_t* __restrict__ blk, int64_t nblk,
                                                             int64_t* __restrict__ counts, int32_t* __restrict__ slot) {
    __shared__ uint64_t s_w[kThreads / 64];
    __shared__ uint32_t s_pre[kThreads / 64][4];
    const int tid = threadIdx.x, lane = tid % 64, wv = tid / 64;
    if (!off) {
        const int64_t upto = blockIdx.x == 0 ? nblk : (int64_t)blockIdx.x;
        uint32_t acc[4] = {0u, 0u, 0u, 0u};
        for (int64_t i = tid; i < upto; i += kThreads) {
            const uint64_t v = blk[i];
#pragma unroll
            for (int k = 0; k < 4; ++k) acc[k] += (uint32_t)((v >> (16 * k)) & 0xffffu);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
#pragma unroll
            for (int o = 32; o >= 1; o /= 2) acc[k] += __shfl_xor(acc[k], o);
            if (lane == 0) s_pre[wv][k] = acc[k];
        }
    }
    const int64_t r0 = (int64_t)blockIdx.x * kPlanRows + 4 * tid;
    uint32_t byte = 0;
    uint64_t c = 0;
    if (r0 < N) {
        byte = tags[r0 / 4];
        for (int i = 0; i < 4 && r0 + i < N; ++i) c += (uint64_t)1 << (16 * tag_at(byte, i));
    }
    uint64_t ex = block_scan_u64(c, s_w) - c;   // rows of each tag before this thread's rows (its barrier also
                                                // orders the s_pre writes above)
    uint32_t ob[4];
    if (off) {
        const uint4 o = off[blockIdx.x];
        ob[0] = o.x; ob[1] = o.y; ob[2] = o.z; ob[3] = o.w;
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            uint32_t t = 0;
            for (int w = 0; w < kThreads / 64; ++w) t += s_pre[w][k];
            ob[k] = blockIdx.x == 0 ? 0u : t;
            if (blockIdx.x == 0 && tid == 0) counts[k] = t;
        }
    }
    if (r0 >= N) return;
    for (int i = 0; i < 4 && r0 + i < N; ++i) {
        const int t = tag_at(byte, i);
        slot[r0 + i] = (int32_t)(ob[t] + (uint32_t)((ex >> (16 * t)) & 0xffffu));
        ex += (uint64_t)1 << (16 * t);
    }
}

// round(x / s) with IEEE-division semantics: the reciprocal fast path of rint_div holds while
// |x / s| < 256 (kvq_internal.h), larger quotients take the division.
__device__ __forceinline__ float rint_q(float x, float s, float r) {
    const float y = x * r;
    float n = __builtin_rintf(y);
    if (__builtin_fabsf(y - n) > 0.4999f || __builtin_fabsf(y) >= 255.0f) n = __builtin_rintf(x / s);
    return n;
}

// reductions over the LPR lanes of a row
template <int LPR>
__device__ __forceinline__ float row_max(float v) { return lane_group_reduce<LPR, true>(v); }
template <int LPR>
__device__ __forceinline__ float row_min(float v) { return lane_group_reduce<LPR, false>(v); }

// Rows of a block share a wave when a row is narrower than a wave (LPR < 64).  The block's ROWS
// rows (at most 64) are then sorted by tag, stably, by one wave: position q of the sorted order
// holds row ts.perm[q] of the block with its tag ts.tag[q] and pool slot ts.slot[q] (rows past N
// last, as tag 0 with slot -1).  The wave loads the rows' tags and slots together, so the block
// waits on memory once before the pool words.  The block still reads and writes its own
// contiguous rows; only their order inside it changes, so a wave runs one precision's code
// for all its rows but at the tag boundaries.
// Blocks of more than 64 rows are sorted in runs of 64, one wave per run (a wave's positions
// never straddle two runs).
template <int ROWS>
struct TagSortLds {
    uint8_t perm[ROWS], tag[ROWS];
    int32_t slot[ROWS];
};
template <int ROWS>
__device__ __forceinline__ void block_tag_sort(const kvq_mixed_store& m, int64_t base, TagSortLds<ROWS>& ts) {
    static_assert(ROWS <= 64 || (ROWS % 64 == 0 && ROWS / 64 <= kThreads / 64), "one wave per run of 64 rows");
    const int tid = threadIdx.x, lane = tid % 64, run = tid / 64;
    if (run * 64 < ROWS) {
        const int rl = run * 64 + lane;   // row of the block
        const int64_t r = base + rl;
        const bool valid = rl < ROWS && r < m.N;
        // both loads before either value is used: one round trip
        uint32_t byte = 0;
        int32_t k = -1;
        if (valid) {
            byte = m.tags[r / 4];
            k = m.slot[r];
        }
        const int t = valid ? tag_at(byte, (int)(r % 4)) : 4;
        const uint64_t b0 = __ballot(t == 0), b1 = __ballot(t == 1), b2 = __ballot(t == 2), b3 = __ballot(t == 3);
        const int c0 = __popcll(b0), c1 = __popcll(b1), c2 = __popcll(b2), c3 = __popcll(b3);
        const uint64_t mine = t == 0 ? b0 : t == 1 ? b1 : t == 2 ? b2 : t == 3 ? b3 : ~(b0 | b1 | b2 | b3);
        const int off = t == 0 ? 0 : t == 1 ? c0 : t == 2 ? c0 + c1 : t == 3 ? c0 + c1 + c2 : c0 + c1 + c2 + c3;
        const int pos = run * 64 + off + __popcll(mine & ((1ull << lane) - 1ull));
        if (rl < ROWS) {
            ts.perm[pos] = (uint8_t)rl;
            ts.tag[pos] = (uint8_t)(valid ? t : 0);
            ts.slot[pos] = k;
        }
    }
    __syncthreads();
}

// Rows per lane group (NR) of the quantizer and dequantizer: rows of at most 512 channels take
// four passes, so a block waits on memory for all of its rows at once (eight passes measured
// slower: the dequantizer's registers then allow 5 waves per SIMD instead of 8).
template <int LPR, int NCH>
constexpr int mixed_passes() { return NCH == 1 ? 4 : 1; }

// One row: LPR lanes, NCH chunks of 8 channels per lane (C = 8 * LPR * NCH), tag t, pool row k.
template <int LPR, int NCH>
__device__ __forceinline__ void quant_row(const kvq_mixed_store& m, const uint4 (&raw)[NCH], int t, int64_t k,
                                          int lane) {
    const int64_t C = m.C;
    const bool fits = k >= 0 && k < cap_of(m, t);
    if (t == 3) {
        if (!fits) return;
#pragma unroll
        for (int j = 0; j < NCH; ++j) *reinterpret_cast<uint4*>(m.x16 + k * C + 8 * (lane + LPR * j)) = raw[j];
        return;
    }
    float v[NCH][8];
#pragma unroll
    for (int j = 0; j < NCH; ++j) unpack8(raw[j], v[j]);
    // Codes leave as bytes of offset binary (q + 2^(bits-1), made by v_cvt_pk_u8_f32 from exact
    // integers) and become two's complement with one xor per word.  The reciprocal only feeds the
    // fast paths of rint_q / rint_div, whose window (|x * r - x / s| below 1e-4 while
    // |x / s| < 256) also covers the hardware reciprocal's 1-ulp error.
    if (t == 2) {
        float mn = FLT_MAX, mx = -FLT_MAX;
#pragma unroll
        for (int j = 0; j < NCH; ++j) minmax8(v[j], mn, mx);
        mn = row_min<LPR>(mn);
        mx = row_max<LPR>(mx);
        const float range = vmax2(mx - mn, 1e-8f);
        const float s = range / 255.0f;
        const float zr = __builtin_rintf(-128.0f - mn / s);
        const float z = vclamp(zr, -128.0f, 127.0f);
        const float rs = __builtin_amdgcn_rcpf(s);
        if (!fits) return;
        if (lane == 0) {
            m.s8[k] = s;
            m.z8[k] = (int8_t)(int)z;
        }
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            float u[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) u[e] = vclamp(rint_q(v[j][e], s, rs) + z, -128.0f, 127.0f) + 128.0f;
            uint32_t w0 = 0, w1 = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                w0 = __builtin_amdgcn_cvt_pk_u8_f32(u[e], e, w0);
                w1 = __builtin_amdgcn_cvt_pk_u8_f32(u[e + 4], e, w1);
            }
            *reinterpret_cast<uint2*>(m.q8 + k * C + 8 * (lane + LPR * j)) =
                make_uint2(w0 ^ 0x80808080u, w1 ^ 0x80808080u);
        }
        return;
    }
    // 2 or 4 bits, symmetric: |x / s| <= qmax, so rint_div's fast path always applies
    float am = 0.0f;
#pragma unroll
    for (int j = 0; j < NCH; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) am = vmax2(am, __builtin_fabsf(v[j][e]));
    am = row_max<LPR>(am);
    const float qmax = t == 0 ? 1.0f : 7.0f;
    const float s = vmax2(am, 1e-8f) / qmax;
    const float rs = __builtin_amdgcn_rcpf(s);
    if (!fits) return;
    if (lane == 0) (t == 0 ? m.s2 : m.s4)[k] = s;
    const float off = qmax + 1.0f;   // 2 or 8
    // no clip: |x| <= max|x| and s = fl(max|x| / qmax) (or the floor's larger s) give
    // |x / s| <= qmax (1 + 2^-23), which rounds into [-qmax, qmax]
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        float u[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) u[e] = rint_div(v[j][e], s, rs) + off;
        uint32_t even = 0, odd = 0;   // bytes: elements 0 2 4 6 and 1 3 5 7
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            even = __builtin_amdgcn_cvt_pk_u8_f32(u[2 * e], e, even);
            odd = __builtin_amdgcn_cvt_pk_u8_f32(u[2 * e + 1], e, odd);
        }
        const int c0 = 8 * (lane + LPR * j);
        if (t == 0) {
            // byte i = c(2i) | c(2i+1) << 2; then the four 4-bit bytes close up into 16 bits
            const uint32_t b = even | (odd << 2);
            const uint32_t b2 = (b | (b >> 4)) & 0x00ff00ffu;
            *reinterpret_cast<uint16_t*>(m.q2 + k * (C / 4) + c0 / 4) = (uint16_t)((b2 | (b2 >> 8)) ^ 0xaaaau);
        } else {
            *reinterpret_cast<uint32_t*>(m.q4 + k * (C / 2) + c0 / 2) = (even | (odd << 4)) ^ 0x88888888u;
        }
    }
}

// Rows of a block: NR passes of RPB rows (NR = 4 for rows of at most 512 channels), the block's
// rows in tag order when several rows share a wave; every row's chunks, tag and slot are loaded
// before any row is processed.  Rows beyond N are skipped as a whole (uniform over the row's lanes).
template <int LPR, int NCH>
__global__ void __launch_bounds__(kThreads) mixed_quant_kernel(const uint16_t* __restrict__ x,
                                                              const kvq_mixed_store m_arg) {
    const kvq_mixed_store m = store_in_sregs(m_arg);
    constexpr int RPB = kThreads / LPR, NR = mixed_passes<LPR, NCH>();
    constexpr int ROWS = RPB * NR, RPW = 64 / LPR;   // rows per block, rows per wave per pass
    constexpr bool SORT = LPR < 64;
    __shared__ TagSortLds<SORT ? ROWS : 1> s_ts;
    const int tid = threadIdx.x, lane = tid % LPR, lg = tid / LPR;
    const int64_t base = (int64_t)blockIdx.x * ROWS;
    if constexpr (SORT) block_tag_sort<ROWS>(m, base, s_ts);
    // sorted position of pass i of lane group lg: a wave takes RPW * NR consecutive positions
    auto pos = [&](int i) -> int { return (lg / RPW) * (RPW * NR) + i * RPW + lg % RPW; };
    auto row = [&](int i) -> int64_t {
        if constexpr (SORT) return base + s_ts.perm[pos(i)];
        else return base + lg + (int64_t)RPB * i;
    };
    uint4 raw[NR][NCH];
    int tg[NR];
    int64_t kk[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        const int64_t r = min(row(i), m.N - 1);
#pragma unroll
        for (int j = 0; j < NCH; ++j) raw[i][j] = *reinterpret_cast<const uint4*>(x + r * m.C + 8 * (lane + LPR * j));
        if constexpr (SORT) {
            tg[i] = s_ts.tag[pos(i)];
            kk[i] = s_ts.slot[pos(i)];
        } else {
            tg[i] = tag_at(m.tags[r / 4], (int)(r % 4));
            kk[i] = m.slot[r];
        }
    }
#pragma unroll
    for (int i = 0; i < NR; ++i)
        if (row(i) < m.N) quant_row<LPR, NCH>(m, raw[i], tg[i], kk[i], lane);
}

// Dequantization: NR passes of RPB rows per block in the quantizer's order; every row's tag and
// slot first, then every row's pool words, then the arithmetic and the stores.
template <int NCH>
struct RowWords {
    uint4 w[NCH];   // 16-bit rows: 8 bf16; 8 bits: .x .y codes; 4 bits: .x; 2 bits: .x low half
    float s, z;
};

template <int LPR, int NCH>
__device__ __forceinline__ void load_row_words(const kvq_mixed_store& m, int t, int64_t k, int lane, RowWords<NCH>& rw) {
    const int64_t C = m.C;
    const bool fits = k >= 0 && k < cap_of(m, t);
    const int64_t kc = fits ? k : 0;
    rw.s = 0.0f;
    rw.z = 0.0f;
    if (!fits) return;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        const int c0 = 8 * (lane + LPR * j);
        if (t == 3) {
            rw.w[j] = *reinterpret_cast<const uint4*>(m.x16 + kc * C + c0);
        } else if (t == 2) {
            const uint2 q = *reinterpret_cast<const uint2*>(m.q8 + kc * C + c0);
            rw.w[j] = make_uint4(q.x, q.y, 0u, 0u);
        } else if (t == 1) {
            rw.w[j] = make_uint4(*reinterpret_cast<const uint32_t*>(m.q4 + kc * (C / 2) + c0 / 2), 0u, 0u, 0u);
        } else {
            rw.w[j] = make_uint4(*reinterpret_cast<const uint16_t*>(m.q2 + kc * (C / 4) + c0 / 4), 0u, 0u, 0u);
        }
    }
    if (t == 2) {
        rw.s = m.s8[kc];
        rw.z = (float)m.z8[kc];
    } else if (t < 2) {
        rw.s = (t == 0 ? m.s2 : m.s4)[kc];
    }
}

// Rows of one chunk per lane (C <= 512): one 16-byte load per lane whatever the tag.  Each lane
// loads the aligned 16 bytes of its row that hold its 8 codes (the lanes of a 2-, 4- or 8-bit row
// share chunks, and the wave's load still touches each line once) and picks its bytes out with
// selects.  The tag then decides addresses and arithmetic only: loads in branches of their own
// per tag would share registers, and each would wait for the one before it.  The loads of every
// row are issued (row_words_load) before any value is used (row_words_finish).
struct RawWords {
    uint4 w;
    float s;
    int z;
    bool fits;
};
// safe: a readable 16-byte-aligned address of at least 16 bytes; rows that do not fit their pool
// (or whose tag has no scale or zero point) load from it, so no load is conditional and none
// needs a merge with a default value (which would make the next load wait for it)
__device__ __forceinline__ RawWords row_words_load(const kvq_mixed_store& m, int t, int64_t k, int lane,
                                                   uintptr_t safe) {
    typedef __attribute__((address_space(1))) const u32x4_t gu4;
    typedef __attribute__((address_space(1))) const float gf32;
    typedef __attribute__((address_space(1))) const int8_t gi8;
    const bool fits = k >= 0 && k < cap_of(m, t);
    const int sh = t == 0 ? 1 : t == 1 ? 2 : t == 2 ? 3 : 4;   // log2 of the bits per value
    const int64_t rowbytes = (m.C << sh) >> 3;
    const int boff = lane << sh;                                 // first byte of the lane's codes
    // the candidates pass through empty asm statements: a select among fields of one struct may
    // otherwise be rebuilt as an indexed load from a stack copy of it
    uint64_t q2 = (uintptr_t)m.q2, q4 = (uintptr_t)m.q4, q8 = (uintptr_t)m.q8, x16 = (uintptr_t)m.x16;
    uint64_t s2 = (uintptr_t)m.s2, s4 = (uintptr_t)m.s4, s8 = (uintptr_t)m.s8, z8 = (uintptr_t)m.z8;
    asm volatile("" : "+s"(q2), "+s"(q4), "+s"(q8), "+s"(x16));
    asm volatile("" : "+s"(s2), "+s"(s4), "+s"(s8), "+s"(z8));
    const uintptr_t base = t == 0 ? q2 : t == 1 ? q4 : t == 2 ? q8 : x16;
    const uintptr_t sbase = t == 0 ? s2 : t == 1 ? s4 : s8;
    const uintptr_t wa = fits ? base + k * rowbytes + (boff & ~15) : safe;
    const uintptr_t sa = fits && t < 3 ? sbase + 4 * k : safe;
    const uintptr_t za = fits && t == 2 ? z8 + k : safe;
    RawWords r;
    const u32x4_t w = *reinterpret_cast<gu4*>(wa);
    r.w = make_uint4(w.x, w.y, w.z, w.w);
    r.s = *reinterpret_cast<gf32*>(sa);
    r.z = *reinterpret_cast<gi8*>(za);
    r.fits = fits;
    return r;
}
__device__ __forceinline__ void row_words_finish(const RawWords& r, int t, int lane, RowWords<1>& rw) {
    const int sh = t == 0 ? 1 : t == 1 ? 2 : t == 2 ? 3 : 4;
    const int o = (lane << sh) & 15;   // 0 for 16-bit rows, 0 or 8 for 8-bit, a multiple of 4 or 2 below
    const uint4 w = r.fits ? r.w : make_uint4(0u, 0u, 0u, 0u);
    const uint32_t d0 = o < 4 ? w.x : o < 8 ? w.y : o < 12 ? w.z : w.w;
    const uint32_t d1 = o < 8 ? w.y : w.w;
    rw.w[0] = t == 3 ? w : t == 2 ? make_uint4(d0, d1, 0u, 0u)
            : make_uint4(t == 1 ? d0 : (d0 >> (8 * (o & 3))) & 0xffffu, 0u, 0u, 0u);
    rw.s = r.fits && t < 3 ? r.s : 0.0f;
    rw.z = r.fits && t == 2 ? (float)r.z : 0.0f;
}

template <int LPR, int NCH, int OT>
__device__ __forceinline__ void dequant_row(const kvq_mixed_store& m, const RowWords<NCH>& rw, int t, bool fits,
                                            int64_t r, int lane, void* out) {
    const int64_t C = m.C;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        const int c0 = 8 * (lane + LPR * j);
        float v[8];
        if (!fits) {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = 0.0f;
        } else if (t == 3) {
            unpack8(rw.w[j], v);
        } else if (t == 2) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int q = (int)(int8_t)(((e < 4 ? rw.w[j].x : rw.w[j].y) >> (8 * (e % 4))) & 0xffu);
                v[e] = ((float)q - rw.z) * rw.s;
            }
        } else if (t == 1) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int q = ((int)((rw.w[j].x >> (4 * e)) & 15u) ^ 8) - 8;   // 4-bit two's complement
                v[e] = (float)q * rw.s;
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int q = ((int)((rw.w[j].x >> (2 * e)) & 3u) ^ 2) - 2;    // 2-bit two's complement
                v[e] = (float)q * rw.s;
            }
        }
        if constexpr (OT == KVQ_FP32) {
            float* p = static_cast<float*>(out) + r * C + c0;
            *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
            *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
        } else {
            *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + r * C + c0) =
                make_uint4(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]), pack_bf2(v[4], v[5]), pack_bf2(v[6], v[7]));
        }
    }
}

template <int LPR, int NCH, int OT>
__global__ void __launch_bounds__(kThreads) mixed_dequant_kernel(const kvq_mixed_store m_arg,
                                                                void* __restrict__ out) {
    const kvq_mixed_store m = store_in_sregs(m_arg);
    constexpr int RPB = kThreads / LPR, NR = mixed_passes<LPR, NCH>();
    constexpr int ROWS = RPB * NR, RPW = 64 / LPR;
    constexpr bool SORT = LPR < 64;
    __shared__ TagSortLds<SORT ? ROWS : 1> s_ts;
    const int tid = threadIdx.x, lane = tid % LPR, lg = tid / LPR;
    const int64_t base = (int64_t)blockIdx.x * ROWS;
    const int64_t rb = base + lg;
    if constexpr (NCH > 4) {
        // wide rows (C >= 4096): four chunks at a time, so the words of a row do not all live at once
        if (rb >= m.N) return;
        const int t = tag_at(m.tags[rb / 4], (int)(rb % 4));
        const int64_t k = m.slot[rb];
        const bool fits = k >= 0 && k < cap_of(m, t);
        kvq_mixed_store mq = m;
#pragma unroll 1
        for (int j0 = 0; j0 < NCH; j0 += 4) {
            // a view of chunks j0 .. j0+3 as a 4-chunk row shifted by 8 * LPR * j0 channels
            RowWords<4> rw;
            const int64_t shift = (int64_t)8 * LPR * j0;
            mq.x16 = m.x16 ? m.x16 + shift : nullptr;
            mq.q8 = m.q8 ? m.q8 + shift : nullptr;
            mq.q4 = m.q4 ? m.q4 + shift / 2 : nullptr;
            mq.q2 = m.q2 ? m.q2 + shift / 4 : nullptr;
            load_row_words<LPR, 4>(mq, t, k, lane, rw);
            dequant_row<LPR, 4, OT>(mq, rw, t, fits, rb, lane,
                                    OT == KVQ_FP32 ? (void*)(static_cast<float*>(out) + shift)
                                                   : (void*)(static_cast<uint16_t*>(out) + shift));
        }
        return;
    }
    if constexpr (SORT) block_tag_sort<ROWS>(m, base, s_ts);
    auto pos = [&](int i) -> int { return (lg / RPW) * (RPW * NR) + i * RPW + lg % RPW; };
    auto row = [&](int i) -> int64_t {
        if constexpr (SORT) return base + s_ts.perm[pos(i)];
        else return rb + (int64_t)RPB * i;
    };
    int tg[NR];
    int64_t kk[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        if constexpr (SORT) {
            tg[i] = s_ts.tag[pos(i)];
            kk[i] = s_ts.slot[pos(i)];
        } else {
            const int64_t r = min(row(i), m.N - 1);
            tg[i] = tag_at(m.tags[r / 4], (int)(r % 4));
            kk[i] = m.slot[r];
        }
    }
    RowWords<NCH> rw[NR];
    if constexpr (NCH == 1) {
        RawWords raw[NR];
#pragma unroll
        for (int i = 0; i < NR; ++i) raw[i] = row_words_load(m, tg[i], kk[i], lane, (uintptr_t)out);
#pragma unroll
        for (int i = 0; i < NR; ++i) row_words_finish(raw[i], tg[i], lane, rw[i]);
    } else {
#pragma unroll
        for (int i = 0; i < NR; ++i) load_row_words<LPR, NCH>(m, tg[i], kk[i], lane, rw[i]);
    }
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        const int64_t r = row(i);
        if (r < m.N)
            dequant_row<LPR, NCH, OT>(m, rw[i], tg[i], kk[i] >= 0 && kk[i] < cap_of(m, tg[i]), r, lane, out);
    }
}

// C = 8 * LPR * NCH with LPR = min(C / 8, 64)
#define KVQ_MIXED_DISPATCH(C, LAUNCH)                      \
    do {                                                   \
        switch (C) {                                       \
            case 64: LAUNCH(8, 1); break;                  \
            case 128: LAUNCH(16, 1); break;                \
            case 256: LAUNCH(32, 1); break;                \
            case 512: LAUNCH(64, 1); break;                \
            case 1024: LAUNCH(64, 2); break;               \
            case 2048: LAUNCH(64, 4); break;               \
            case 4096: LAUNCH(64, 8); break;               \
            default: LAUNCH(64, 16); break;                \
        }                                                  \
    } while (0)

int check_store(const kvq_mixed_store* m, const char* name, bool need_pools) {
    KVQ_REQUIRE(m, "%s: NULL store descriptor", name);
    KVQ_REQUIRE(m->N >= 1 && m->N < ((int64_t)1 << 31), "%s: need 1 <= N < 2^31", name);
    KVQ_REQUIRE(m->C == 64 || m->C == 128 || m->C == 256 || m->C == 512 || m->C == 1024 || m->C == 2048 ||
                    m->C == 4096 || m->C == 8192,
                "%s: C must be a power of two in [64, 8192] (got %lld)", name, (long long)m->C);
    KVQ_REQUIRE(m->tags && m->slot, "%s: NULL tags or slot", name);
    for (int i = 0; i < 4; ++i) KVQ_REQUIRE(m->cap[i] >= 0, "%s: negative pool capacity", name);
    if (need_pools) {
        KVQ_REQUIRE(m->cap[0] == 0 || (m->q2 && m->s2), "%s: NULL 2-bit pool", name);
        KVQ_REQUIRE(m->cap[1] == 0 || (m->q4 && m->s4), "%s: NULL 4-bit pool", name);
        KVQ_REQUIRE(m->cap[2] == 0 || (m->q8 && m->s8 && m->z8), "%s: NULL 8-bit pool", name);
        KVQ_REQUIRE(m->cap[3] == 0 || m->x16, "%s: NULL 16-bit pool", name);
        KVQ_REQUIRE_ALIGNED(m->q2, "q2");
        KVQ_REQUIRE_ALIGNED(m->q4, "q4");
        KVQ_REQUIRE_ALIGNED(m->q8, "q8");
        KVQ_REQUIRE_ALIGNED(m->x16, "x16");
    }
    return KVQ_OK;
}

}  // namespace
}  // namespace kvq

extern "C" {

size_t kvq_mixed_plan_ws(int64_t N) {
    if (N < 1) return 0;
    const int64_t nblk = kvq::cdiv(N, kvq::kPlanRows);
    return (size_t)(kvq::cdiv(nblk * 8, 16) * 16 + nblk * 16);
}

int kvq_mixed_plan(const uint8_t* tags, int64_t N, int32_t* slot, int64_t* counts, void* ws, size_t ws_bytes,
                   kvq_stream stream) {
    KVQ_REQUIRE(N >= 1 && N < ((int64_t)1 << 31), "kvq_mixed_plan: need 1 <= N < 2^31");
    KVQ_REQUIRE(tags && slot && counts, "kvq_mixed_plan: NULL tags, slot or counts");
    KVQ_REQUIRE(ws && ws_bytes >= kvq_mixed_plan_ws(N), "kvq_mixed_plan: workspace of %zu bytes needed",
                kvq_mixed_plan_ws(N));
    KVQ_REQUIRE_ALIGNED(ws, "ws");
    const int64_t nblk = kvq::cdiv(N, kvq::kPlanRows);
    uint64_t* blk = static_cast<uint64_t*>(ws);
    uint4* off = reinterpret_cast<uint4*>(static_cast<char*>(ws) + kvq::cdiv(nblk * 8, 16) * 16);
    KVQ_REQUIRE(kvq::cdiv(nblk * 8, 16) * 16 + nblk * 16 <= (int64_t)ws_bytes, "kvq_mixed_plan: workspace too small");
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(kvq::mixed_count_kernel, dim3((unsigned)nblk), dim3(kvq::kThreads), 0, st, tags, N, blk);
    const bool self_prefix = nblk <= kvq::kSelfPrefixBlocks;
    if (!self_prefix) hipLaunchKernelGGL(kvq::mixed_scan_kernel, dim3(1), dim3(1024), 0, st, blk, off, nblk, counts);
    hipLaunchKernelGGL(kvq::mixed_slot_kernel, dim3((unsigned)nblk), dim3(kvq::kThreads), 0, st, tags, N,
                       self_prefix ? nullptr : static_cast<const uint4*>(off), static_cast<const uint64_t*>(blk), nblk,
                       counts, slot);
    return kvq::launch_status("kvq_mixed_plan");
}

int kvq_mixed_quant(const void* x, const kvq_mixed_store* m, kvq_stream stream) {
    const int rc = kvq::check_store(m, "kvq_mixed_quant", true);
    if (rc) return rc;
    KVQ_REQUIRE(x, "kvq_mixed_quant: NULL x");
    KVQ_REQUIRE_ALIGNED(x, "x");
    hipStream_t st = static_cast<hipStream_t>(stream);
    const uint16_t* xp = static_cast<const uint16_t*>(x);
#define KVQ_MQ(LPR, NCH)                                                                                    \
    hipLaunchKernelGGL((kvq::mixed_quant_kernel<LPR, NCH>),                                                 \
                       dim3((unsigned)kvq::cdiv(m->N, (kvq::kThreads / LPR) * kvq::mixed_passes<LPR, NCH>())),                \
                       dim3(kvq::kThreads), 0, st, xp, *m)
    KVQ_MIXED_DISPATCH(m->C, KVQ_MQ);
#undef KVQ_MQ
    return kvq::launch_status("kvq_mixed_quant");
}

int kvq_mixed_dequant(const kvq_mixed_store* m, void* out, int ot, kvq_stream stream) {
    const int rc = kvq::check_store(m, "kvq_mixed_dequant", true);
    if (rc) return rc;
    KVQ_REQUIRE(out, "kvq_mixed_dequant: NULL out");
    KVQ_REQUIRE(ot == KVQ_FP32 || ot == KVQ_BF16, "kvq_mixed_dequant: ot must be KVQ_FP32 or KVQ_BF16");
    KVQ_REQUIRE_ALIGNED(out, "out");
    hipStream_t st = static_cast<hipStream_t>(stream);
#define KVQ_MD(LPR, NCH)                                                                                       \
    do {                                                                                                       \
        const dim3 grid((unsigned)kvq::cdiv(m->N, (kvq::kThreads / LPR) * kvq::mixed_passes<LPR, NCH>()));               \
        if (ot == KVQ_FP32)                                                                                    \
            hipLaunchKernelGGL((kvq::mixed_dequant_kernel<LPR, NCH, KVQ_FP32>), grid, dim3(kvq::kThreads), 0, st, \
                               *m, out);                                                                       \
        else                                                                                                   \
            hipLaunchKernelGGL((kvq::mixed_dequant_kernel<LPR, NCH, KVQ_BF16>), grid, dim3(kvq::kThreads), 0, st, \
                               *m, out);                                                                       \
    } while (0)
    KVQ_MIXED_DISPATCH(m->C, KVQ_MD);
#undef KVQ_MD
    return kvq::launch_status("kvq_mixed_dequant");
}

int kvq_mixed_bytes(const int64_t counts[4], int64_t N, int64_t C, uint64_t out[3]) {
    KVQ_REQUIRE(counts && out, "kvq_mixed_bytes: NULL pointer");
    KVQ_REQUIRE(N >= 0 && C >= 8 && C % 8 == 0, "kvq_mixed_bytes: invalid N or C");
    for (int i = 0; i < 4; ++i) KVQ_REQUIRE(counts[i] >= 0, "kvq_mixed_bytes: negative count");
    out[0] = (uint64_t)(counts[0] * (C / 4) + counts[1] * (C / 2) + counts[2] * C + counts[3] * C * 2);
    out[1] = (uint64_t)(counts[0] * 4 + counts[1] * 4 + counts[2] * 5);
    out[2] = (uint64_t)((N + 3) / 4);
    return KVQ_OK;
}

}  // extern "C"
