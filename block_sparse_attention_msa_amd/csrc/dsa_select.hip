// dsa_select.hip -- DSA lightning-indexer token selection.
//
// "deepseek2 : GLM-DSA sparse attention (lightning indexer), --dsa off by
// default", What this does: each query is scored against every (Hadamard-
// rotated, F16-cached) indexer key and keeps its top-k highest-scoring keys.
// Readings: one score per (query, key) = fp16 dot product accumulated in f32;
// keys j <= pos only; k = min(top_k, pos + 1); ties to the lower token id.
//
// Kernel 1 streams the fp16 key cache once with 128-bit loads (a 16-lane DPP
// row per 256-byte key row, v_dot2 on fp16 pairs) and writes the f32 scores.
// Its multi-head form (same pull request, review thread: one score per
// indexer head, an element-wise product with the head weights and a
// reduction over the heads before the top-k; the reduction is read as the
// lightning indexer's sum over heads of weight x ReLU(q_h . k)) contracts 16
// keys at a time against all heads on the fp16 matrix cores.
// Kernel 2 is an exact radix select on order-preserving u32 keys (digits of
// 12, 12 and 8 bits) that finds the k-th largest key T, then an order-
// preserving compaction writes every key > T and the lowest-id keys == T, so
// the output is already in ascending id order and unique.  Contexts of up to
// 65536 keys run it with every key in registers (one burst of loads, no
// further pass over memory); longer ones stream the scores for each pass.
#include "common.hpp"

namespace msa {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

constexpr int kScoreKeysPerWg = 1024;
constexpr int kScoreUnroll = 8;
constexpr int kSelThreads = 1024;

__device__ __forceinline__ float dot8_f16(const u32x4& q, const u32x4& k) {
    float d = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        // copy the element out first: a bit-cast of a vector-element lvalue
        // reads element 0 whatever the index
        const uint32_t qe = q[e], ke = k[e];
        d = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, qe), __builtin_bit_cast(half2_t, ke), d, false);
    }
    return d;
}

__global__ __launch_bounds__(256) void dsa_score_kernel(const uint16_t* __restrict__ dsa_k, Pager pg,
                                                        const uint16_t* __restrict__ q_idx,
                                                        const int32_t* __restrict__ q_stream,
                                                        const int32_t* __restrict__ q_pos,
                                                        float* __restrict__ scores, int64_t stride) {
    const int64_t i = blockIdx.y;
    const int p = q_pos[i];
    const int j_wg = blockIdx.x * kScoreKeysPerWg;
    if (j_wg > p) return;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: scalar table reads
    const int r = lane >> 4;     // key row within a group of four
    const int c = lane & 15;     // 16-byte column (8 fp16 dims)
    const u32x4 q = *reinterpret_cast<const u32x4*>(q_idx + i * kIdxDim + 8 * c);
    const int64_t s = q_stream[i];
    float* out = scores + i * stride;
    const int j_begin = j_wg + wave * (kScoreKeysPerWg / 4);
    const int j_end = min(j_begin + kScoreKeysPerWg / 4, p + 1);
    static_assert(kBlock % (4 * kScoreUnroll) == 0, "an iteration's keys lie in one 128-key block");
    for (int j0 = j_begin; j0 < j_end; j0 += 4 * kScoreUnroll) {
        // keys j0 .. j0 + 31 (and p >= j0) share one block: one row lookup
        const int64_t rb = pg.block_row_uniform(s, j0 / kBlock);
        const int jb = j0 & ~(kBlock - 1);
        u32x4 kr[kScoreUnroll];
#pragma unroll
        for (int u = 0; u < kScoreUnroll; ++u) {
            int j = j0 + 4 * u + r;
            j = min(j, p);                                   // rows past p are never written
            kr[u] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4*>(dsa_k + (rb + (j - jb)) * kIdxDim + 8 * c));
        }
#pragma unroll
        for (int u = 0; u < kScoreUnroll; ++u) {
            const float d = row16_sum(dot8_f16(q, kr[u]));
            const int j = j0 + 4 * u + r;
            if (c == 0 && j < j_end) out[j] = d;
        }
    }
}

// Multi-head scores, H = 16 * kTiles heads.  Per 16-key group a wave forms
// D[head][key] = Q K^T with v_mfma_f32_16x16x32_f16 (heads are the M side,
// keys the N side; four 32-dim slices per head tile), applies ReLU and the
// head weights to its 4 rows per tile in registers, and sums the heads with
// two cross-row swaps, after which every lane holds its key's score.  A lane
// reads 4 x 16 bytes of one key row (dims 32c + 8 * (lane / 16) ..), so one
// load instruction covers a contiguous 64-byte piece of 16 rows.  A wave
// walks 1024 keys, 64 (16 KiB) per step, with the next step's keys loading
// while the current step's products run (one workgroup of 4 waves per 4096
// keys of a query).  Measured on 16 x 65536 keys, 32 heads: 48 us, as fast as
// a plain read of the same 268 MB (45-50 us); shorter waves (64-512 keys) or
// no prefetch ran 49-60 us.
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
constexpr int kMhWaves = 4;
constexpr int kMhKeysPerWave = 1024;
constexpr int kMhKeysPerWg = kMhWaves * kMhKeysPerWave;
constexpr int kMhGroups = 4;                 // 16-key groups per step
constexpr int kMhStep = 16 * kMhGroups;
static_assert(kBlock % kMhStep == 0, "a step's keys lie in one 128-key block");

template <int kTiles>
__global__ __launch_bounds__(64 * kMhWaves) void dsa_score_heads_kernel(
    const uint16_t* __restrict__ dsa_k, Pager pg, const uint16_t* __restrict__ q_idx_h,
    const float* __restrict__ head_w, const int32_t* __restrict__ q_stream,
    const int32_t* __restrict__ q_pos, float* __restrict__ scores, int64_t stride) {
    constexpr int kHeads = 16 * kTiles;
    const int64_t i = blockIdx.y;
    const int p = q_pos[i];
    const int j_wg = blockIdx.x * kMhKeysPerWg;
    if (j_wg > p) return;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: scalar table reads
    const int l16 = lane & 15;
    const int l4 = lane >> 4;
    // A operand: head 16t + l16, dims 32c + 8 * l4 .. + 7
    f16x8 qa[kTiles][4];
    // weights of the D rows this lane holds: heads 16t + 4 * l4 + r
    f32x4 wr[kTiles];
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
        const uint16_t* qh = q_idx_h + (i * kHeads + 16 * t + l16) * kIdxDim + 8 * l4;
#pragma unroll
        for (int c = 0; c < 4; ++c) qa[t][c] = *reinterpret_cast<const f16x8*>(qh + 32 * c);
        wr[t] = *reinterpret_cast<const f32x4*>(head_w + i * kHeads + 16 * t + 4 * l4);
    }
    const int64_t s = q_stream[i];
    float* out = scores + i * stride;
    const int j_begin = j_wg + wave * kMhKeysPerWave;
    const int j_end = min(j_begin + kMhKeysPerWave, p + 1);

    auto load = [&](f16x8 (&kb)[kMhGroups][4], int j0) __attribute__((always_inline)) {
        const int64_t rb = pg.block_row_uniform(s, j0 / kBlock);
        const int jb = j0 & ~(kBlock - 1);
#pragma unroll
        for (int u = 0; u < kMhGroups; ++u) {
            const int j = min(j0 + 16 * u + l16, p);           // rows past p are never written
            const f16x8* row = reinterpret_cast<const f16x8*>(dsa_k + (rb + (j - jb)) * kIdxDim + 8 * l4);
#pragma unroll
            for (int c = 0; c < 4; ++c) kb[u][c] = __builtin_nontemporal_load(row + 4 * c);
        }
    };
    auto compute = [&](const f16x8 (&kb)[kMhGroups][4], int j0) __attribute__((always_inline)) {
        float tot[kMhGroups];
#pragma unroll
        for (int u = 0; u < kMhGroups; ++u) {
            float acc = 0.f;
#pragma unroll
            for (int t = 0; t < kTiles; ++t) {
                f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < 4; ++c) d = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[t][c], kb[u][c], d, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc = __builtin_fmaf(wr[t][r], fmaxf(d[r], 0.f), acc);
            }
            tot[u] = sum_xor32(sum_xor16(acc));               // all heads: key j0 + 16u + l16
        }
        // lane (l16, l4) writes key j0 + 16 * l4 + l16: 256 contiguous bytes
        float v = tot[0];
#pragma unroll
        for (int u = 1; u < kMhGroups; ++u) v = l4 == u ? tot[u] : v;
        const int j = j0 + 16 * l4 + l16;
        if (j < j_end) out[j] = v;
    };
    // Two register sets: the next step's keys load while this step computes.
    // Each branch holds its load and the products after it, so the wait
    // before the products leaves the prefetch in flight (a load issued on
    // one path only would make the wait at the join drain every load).
    if (j_begin >= j_end) return;
    f16x8 ka[kMhGroups][4], kn[kMhGroups][4];
    load(ka, j_begin);
    for (int j0 = j_begin;; j0 += 2 * kMhStep) {
        if (j0 + kMhStep < j_end) {
            load(kn, j0 + kMhStep);
            __builtin_amdgcn_sched_barrier(0);                // loads issued before the products
            compute(ka, j0);
        } else {
            compute(ka, j0);
            break;
        }
        if (j0 + 2 * kMhStep < j_end) {
            load(ka, j0 + 2 * kMhStep);
            __builtin_amdgcn_sched_barrier(0);
            compute(kn, j0 + kMhStep);
        } else {
            compute(kn, j0 + kMhStep);
            break;
        }
    }
}

// Inclusive prefix sum over the 64 lanes of a wave: row_shr DPP steps inside
// each 16-lane row, then the totals of the lower rows (read from lanes 15,
// 31, 47) are added.
__device__ __forceinline__ int wave_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);    // row_shr:1 (lanes past the row's start read 0)
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);    // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);    // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);    // row_shr:8
    const int r = (threadIdx.x & 63) >> 4;
    const int t0 = __builtin_amdgcn_readlane(x, 15);
    const int t1 = __builtin_amdgcn_readlane(x, 31);
    const int t2 = __builtin_amdgcn_readlane(x, 47);
    return x + (r >= 1 ? t0 : 0) + (r >= 2 ? t1 : 0) + (r >= 3 ? t2 : 0);
}
// Sum over the 64 lanes of a wave (every lane gets it): DPP inside each
// 16-lane row, then the four row totals.
__device__ __forceinline__ int wave_sum(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xf, 0xf, false);     // quad_perm [1,0,3,2]
    x += __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xf, 0xf, false);     // quad_perm [2,3,0,1]
    x += __builtin_amdgcn_update_dpp(0, x, 0x141, 0xf, 0xf, false);    // row_half_mirror
    x += __builtin_amdgcn_update_dpp(0, x, 0x140, 0xf, 0xf, false);    // row_mirror
    return __builtin_amdgcn_readlane(x, 0) + __builtin_amdgcn_readlane(x, 16) +
           __builtin_amdgcn_readlane(x, 32) + __builtin_amdgcn_readlane(x, 48);
}

// Inclusive prefix sum over the kThreads threads of the workgroup: wave
// scans, one barrier, each wave adds the totals of the waves below it.
// With kDone, a final barrier frees wave_sums for the next use (a caller
// that ends in a barrier of its own before reusing it passes false).
template <int kThreads, typename T, bool kDone = true>
__device__ T block_scan(T v, T* wave_sums) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    v = wave_scan(v);
    if (lane == 63) wave_sums[wave] = v;
    __syncthreads();
    T below = T(0);
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) below += w < wave ? wave_sums[w] : T(0);
    if (kDone) __syncthreads();
    return v + below;
}
__device__ int block_inclusive_scan(int v, int* wave_sums) { return block_scan<kSelThreads>(v, wave_sums); }

// Digits of the radix select, most significant first: 12 + 12 + 8 bits.
// Wide first digits spread the (exponent-concentrated) f32 scores over many
// histogram bins, which keeps LDS atomic collisions rare.
constexpr int kDigitBits[3] = {12, 12, 8};
constexpr int kBins = 4096;

// One workgroup of 1024 threads per query, three streaming passes over the
// query's scores (16-byte loads, coalesced across the workgroup):
//  1. histogram of the top 12 key bits -> the digit d1 of the top_k-th
//     largest key T, and how many keys equal to T's prefix are still needed;
//  2. the keys whose top 12 bits equal d1 (the boundary bin, typically ~1% of
//     the keys) are copied with their ids into an LDS candidate list, whose
//     remaining 12 + 8 bits are resolved there;
//  3. an order-preserving compaction in rounds of 16384 consecutive keys emits
//     every key > T and the lowest-id keys == T, ascending.
// A boundary bin larger than the LDS list (heavily tied scores) takes the
// general path, which re-reads the scores for the last two digits.
constexpr int kCandCap = 4096;

// Visits every score j < n as (j, ordered key).  Each thread issues four
// 16-byte loads per batch (j = 4 * (tid + 1024 * r) + c, coalesced across the
// workgroup) before using any of them.
constexpr int kBatch = 4;

template <typename F>
__device__ __forceinline__ void for_each_score(const float* t, int n, F&& f) {
    const int full = n & ~3;
    for (int base = 4 * threadIdx.x; base < full; base += 4 * kSelThreads * kBatch) {
        f32x4 x[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int j = base + 4 * kSelThreads * u;
            x[u] = j < full ? *reinterpret_cast<const f32x4*>(t + j) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int j = base + 4 * kSelThreads * u;
            if (j < full) {
                f(j, ordered_key(x[u].x));
                f(j + 1, ordered_key(x[u].y));
                f(j + 2, ordered_key(x[u].z));
                f(j + 3, ordered_key(x[u].w));
            }
        }
    }
    if (static_cast<int>(threadIdx.x) < n - full) f(full + threadIdx.x, ordered_key(t[full + threadIdx.x]));
}

// Finds the digit (bits `bits` wide) of the rank-`remaining` largest among
// the histogram counts; returns it through s_digit / s_remaining.
template <int kThreads>
__device__ __forceinline__ void pick_digit_t(const int* hist, int bits, int remaining, int* wave_sums,
                                             uint32_t* s_digit, int* s_remaining) {
    constexpr int kPer = kBins / kThreads;
    const int nb = 1 << bits;
    int c[kPer];
    int csum = 0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
        const int dd = kPer * threadIdx.x + e;    // descending bin order
        c[e] = dd < nb ? hist[nb - 1 - dd] : 0;
        csum += c[e];
    }
    const int incl = block_scan<kThreads, int, false>(csum, wave_sums);   // the barrier below frees wave_sums
    if (incl >= remaining && incl - csum < remaining) {
        int before = incl - csum;
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
            if (before + c[e] >= remaining) {
                *s_digit = static_cast<uint32_t>(nb - 1 - (kPer * threadIdx.x + e));
                *s_remaining = remaining - before;
                break;
            }
            before += c[e];
        }
    }
    __syncthreads();
}
__device__ __forceinline__ void pick_digit(const int* hist, int bits, int remaining, int* wave_sums,
                                           uint32_t* s_digit, int* s_remaining) {
    pick_digit_t<kSelThreads>(hist, bits, remaining, wave_sums, s_digit, s_remaining);
}

__global__ __launch_bounds__(kSelThreads) void dsa_topk_kernel(const float* __restrict__ scores,
                                                               int64_t stride,
                                                               const int32_t* __restrict__ q_pos,
                                                               int top_k, int32_t* __restrict__ sel,
                                                               int32_t* __restrict__ n_sel) {
    __shared__ int hist[kBins];
    __shared__ uint32_t cand_key[kCandCap];
    __shared__ int32_t cand_id[kCandCap];
    __shared__ int wave_sums[kSelThreads / 64];
    __shared__ uint32_t s_digit;
    __shared__ int s_remaining;
    __shared__ int s_ncand;
    const int64_t i = blockIdx.x;
    const int tid = threadIdx.x;
    const int n = q_pos[i] + 1;
    const float* t = scores + i * stride;
    int32_t* out = sel + i * top_k;
    if (n <= top_k) {                                   // every visible key is kept
        for (int j = tid; j < top_k; j += kSelThreads) out[j] = j < n ? j : -1;
        if (tid == 0) n_sel[i] = n;
        return;
    }
    // ---- pass 1: top 12 bits over all keys
    for (int b = tid; b < kBins; b += kSelThreads) hist[b] = 0;
    if (tid == 0) s_ncand = 0;
    __syncthreads();
    for_each_score(t, n, [&](int, uint32_t key) { atomicAdd(&hist[key >> 20], 1); });
    __syncthreads();
    pick_digit(hist, 12, top_k, wave_sums, &s_digit, &s_remaining);
    const uint32_t d1 = s_digit;
    int remaining = s_remaining;
    const int bin_count = hist[d1];
    uint32_t prefix = d1 << 20, mask = 0xfff00000u;
    __syncthreads();
    if (bin_count <= kCandCap) {
        // ---- pass 2: gather the boundary bin, resolve the low 20 bits in LDS
        for_each_score(t, n, [&](int j, uint32_t key) {
            if ((key & mask) == prefix) {
                const int slot = atomicAdd(&s_ncand, 1);
                cand_key[slot] = key;
                cand_id[slot] = j;
            }
        });
        __syncthreads();
        const int nc = s_ncand;
#pragma unroll
        for (int pass = 1; pass < 3; ++pass) {
            const int bits = kDigitBits[pass];
            const int shift = pass == 1 ? 8 : 0;
            const uint32_t dmask = (1u << bits) - 1;
            for (int b = tid; b < kBins; b += kSelThreads) hist[b] = 0;
            __syncthreads();
            for (int c = tid; c < nc; c += kSelThreads) {
                const uint32_t key = cand_key[c];
                if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1);
            }
            __syncthreads();
            pick_digit(hist, bits, remaining, wave_sums, &s_digit, &s_remaining);
            prefix |= s_digit << shift;
            mask |= dmask << shift;
            remaining = s_remaining;
            __syncthreads();
        }
    } else {
        // ---- general path: the last two digits over all keys
#pragma unroll
        for (int pass = 1; pass < 3; ++pass) {
            const int bits = kDigitBits[pass];
            const int shift = pass == 1 ? 8 : 0;
            const uint32_t dmask = (1u << bits) - 1;
            for (int b = tid; b < kBins; b += kSelThreads) hist[b] = 0;
            __syncthreads();
            for_each_score(t, n, [&](int, uint32_t key) {
                if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1);
            });
            __syncthreads();
            pick_digit(hist, bits, remaining, wave_sums, &s_digit, &s_remaining);
            prefix |= s_digit << shift;
            mask |= dmask << shift;
            remaining = s_remaining;
            __syncthreads();
        }
    }
    const uint32_t T = prefix;          // the top_k-th largest key; `remaining` keys equal to it are kept
    // ---- pass 3: order-preserving compaction; thread tid takes 16 consecutive
    // keys of each round of 16384
    constexpr int kPer = 16;
    int written = 0, eq_seen = 0;       // running totals over the rounds (uniform)
    for (int base = 0; base < n; base += kPer * kSelThreads) {
        const int j = base + kPer * tid;
        uint32_t key[kPer];
#pragma unroll
        for (int v = 0; v < kPer / 4; ++v) {
            const int jj = j + 4 * v;
            if (jj + 3 < n) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(t + jj);
                key[4 * v] = ordered_key(x.x);
                key[4 * v + 1] = ordered_key(x.y);
                key[4 * v + 2] = ordered_key(x.z);
                key[4 * v + 3] = ordered_key(x.w);
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) key[4 * v + c] = jj + c < n ? ordered_key(t[jj + c]) : 0u;
            }
        }
        int n_eq = 0;
#pragma unroll
        for (int c = 0; c < kPer; ++c) n_eq += (j + c < n) && key[c] == T;
        const int eq_incl = block_inclusive_scan(n_eq, wave_sums);
        int eq_rank = eq_seen + eq_incl - n_eq;      // equal keys before this thread's keys
        uint32_t take = 0;
        int n_take = 0;
#pragma unroll
        for (int c = 0; c < kPer; ++c) {
            const bool in = j + c < n;
            const bool eq = in && key[c] == T;
            const bool tk = (in && key[c] > T) || (eq && eq_rank < remaining);
            eq_rank += eq;
            take |= static_cast<uint32_t>(tk) << c;
            n_take += tk;
        }
        const int take_incl = block_inclusive_scan(n_take, wave_sums);
        int w = written + take_incl - n_take;
#pragma unroll
        for (int c = 0; c < kPer; ++c) {
            if ((take >> c) & 1) {
                if (w < top_k) out[w] = j + c;      // exactly top_k keys qualify; the bound is defensive
                ++w;
            }
        }
        // round totals: the last thread's inclusive values, via the scan's LDS
        if (tid == kSelThreads - 1) {
            wave_sums[0] = eq_incl;
            wave_sums[1] = take_incl;
        }
        __syncthreads();
        eq_seen += wave_sums[0];
        written += wave_sums[1];
        __syncthreads();
    }
    if (tid == 0) n_sel[i] = top_k;
}

// ---------------------------------------------------------------------------
// Contexts of at most 65536 keys: the same selection with every key held in
// registers.  1024 threads; lane l of wave w holds the keys of ids 4096 w +
// 256 r + 4 l + c (round r < 16, c < 4), read in one burst of coalesced
// 16-byte loads (the scores come from other compute units' writes, so each
// pass over memory would cost a full memory latency).  The three digits are
// histogrammed from the registers: the first over eight copies (by lane),
// because the exponent-heavy keys pile into few bins, the next two over a
// list of the keys in the first digit's boundary bin (a block scan of the
// threads' match counts places them; typically a few hundred keys).  The
// compaction counts each wave's keys above T and equal to T (one scan over
// the waves gives each wave its output offset), then walks the rounds in id
// order: ballots of the lanes' keys above and equal to T rank every kept key
// (the kept keys of lower lanes, then the lane's own earlier ones), into an
// LDS copy of the output that is written out coalesced at the end.  No step
// branches per key: a key that is not counted or kept goes to a spare bin or
// slot of its lane instead.
// ---------------------------------------------------------------------------
constexpr int kRegThreads = 1024;
constexpr int kRegWaves = kRegThreads / 64;
constexpr int kRegRounds = 16;
constexpr int kRegPer = 4 * kRegRounds;                   // keys per lane
constexpr int kRegKeys = kRegThreads * kRegPer;           // 65536
constexpr int kHistCopies = 8;
constexpr int kTopKMax = 4096;
constexpr int kCandRegCap = (kHistCopies - 1) * (kBins + 64);   // boundary-bin keys the freed copies hold

__global__ __launch_bounds__(kRegThreads) void dsa_topk_regs_kernel(const float* __restrict__ scores,
                                                                    int64_t stride,
                                                                    const int32_t* __restrict__ q_pos,
                                                                    int top_k, int32_t* __restrict__ sel,
                                                                    int32_t* __restrict__ n_sel) {
    __shared__ int hist[kHistCopies][kBins + 64];    // + one spare bin per lane: where keys past the last go
    __shared__ int32_t ostage[kTopKMax + 64];        // the output, in order (+ one spare slot per lane)
    __shared__ int wave_sums[kRegWaves];
    __shared__ uint32_t wave_tot[kRegWaves];
    __shared__ uint32_t s_digit;
    __shared__ int s_remaining;
    __shared__ uint32_t s_T;
    __shared__ int s_ncand;
    const int64_t i = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int n = q_pos[i] + 1;
    const float* t = scores + i * stride;
    int32_t* out = sel + i * top_k;
    if (n <= top_k) {                                   // every visible key is kept
        for (int j = tid; j < top_k; j += kRegThreads) out[j] = j < n ? j : -1;
        if (tid == 0) n_sel[i] = n;
        return;
    }
    // keys past the last are 0, below the key of every score (that of -inf
    // is 0x007fffff), so they never match a prefix or the threshold.  Every
    // load is unconditional (from inside the row), so that all are in
    // flight together.
    const int base = 4096 * wave + 4 * lane;            // id of this lane's key (r, c): base + 256 r + c
    uint32_t rk[kRegPer];
    const int last4 = static_cast<int>(stride) - 4;    // the row holds stride >= n scores
    {
        f32x4 x[kRegRounds];
#pragma unroll
        for (int r = 0; r < kRegRounds; ++r) x[r] = *reinterpret_cast<const f32x4*>(t + min(base + 256 * r, last4));
        // (a mask, not a select: a select becomes a branch per key with a
        // wait for its load inside, which serialises the loads)
#pragma unroll
        for (int r = 0; r < kRegRounds; ++r)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                rk[4 * r + c] = ordered_key(x[r][c]) & (0u - static_cast<uint32_t>(base + 256 * r + c < n));
    }
    // ---- digit 1: top 12 bits (keys past the last go to the lane's spare bin)
    for (int b = tid; b < kHistCopies * (kBins + 64); b += kRegThreads) (&hist[0][0])[b] = 0;
    __syncthreads();
    {
        int* hc = hist[lane % kHistCopies];
#pragma unroll
        for (int e = 0; e < kRegPer; ++e) {
            const uint32_t key = rk[e];
            atomicAdd(&hc[key != 0u ? static_cast<int>(key >> 20) : kBins + lane], 1);
        }
    }
    __syncthreads();
    for (int b = tid; b < kBins; b += kRegThreads) {
        int sum = 0;
#pragma unroll
        for (int k = 0; k < kHistCopies; ++k) sum += hist[k][b];
        hist[0][b] = sum;
    }
    __syncthreads();
    pick_digit_t<kRegThreads>(hist[0], 12, top_k, wave_sums, &s_digit, &s_remaining);
    uint32_t prefix = s_digit << 20, mask = 0xfff00000u;
    int remaining = s_remaining;
    // ---- digits 2 and 3 (12 and 8 bits) over the keys with the prefix: the
    // boundary bin (typically a few hundred keys) is first copied into a
    // list in the free histogram copies, so each digit histograms the list
    // only; a bin too large for the list takes every key per digit
    uint32_t* cand = reinterpret_cast<uint32_t*>(&hist[1][0]);
    int n_match = 0;
#pragma unroll
    for (int e = 0; e < kRegPer; ++e) n_match += (rk[e] & mask) == prefix;
    const int m_incl = block_scan<kRegThreads>(n_match, wave_sums);
    if (tid == kRegThreads - 1) s_ncand = m_incl;
    __syncthreads();
    const int n_cand = s_ncand;
    if (n_cand <= kCandRegCap) {
        int slot = m_incl - n_match;
#pragma unroll
        for (int e = 0; e < kRegPer; ++e) {
            if ((rk[e] & mask) == prefix) cand[slot++] = rk[e];
        }
    }
#pragma unroll
    for (int pass = 1; pass < 3; ++pass) {
        const int bits = kDigitBits[pass];
        const int shift = pass == 1 ? 8 : 0;
        const uint32_t dmask = (1u << bits) - 1;
        for (int b = tid; b < kBins; b += kRegThreads) hist[0][b] = 0;
        __syncthreads();
        if (n_cand <= kCandRegCap) {               // workgroup-uniform
            for (int c = tid; c < n_cand; c += kRegThreads) {
                const uint32_t key = cand[c];
                if ((key & mask) == prefix) atomicAdd(&hist[0][(key >> shift) & dmask], 1);
            }
        } else {
#pragma unroll
            for (int e = 0; e < kRegPer; ++e) {
                const uint32_t key = rk[e];
                atomicAdd(&hist[0][(key & mask) == prefix ? static_cast<int>((key >> shift) & dmask) : kBins + lane], 1);
            }
        }
        __syncthreads();
        pick_digit_t<kRegThreads>(hist[0], bits, remaining, wave_sums, &s_digit, &s_remaining);
        prefix |= s_digit << shift;
        mask |= dmask << shift;
        remaining = s_remaining;
    }
    const uint32_t T = prefix;          // the top_k-th largest key; `remaining` keys equal to it are kept
    // ---- compaction: each wave's counts, packed as (keys > T) + (keys == T)
    // << 16 (at most 4096 per wave, and below 2^16 summed over the earlier
    // waves)
    uint32_t v = 0;
#pragma unroll
    for (int e = 0; e < kRegPer; ++e) v += (rk[e] > T ? 1u : 0u) + (rk[e] == T ? 0x10000u : 0u);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    if (lane == 0) wave_tot[wave] = v;
    if (tid == 0) s_T = T;
    __syncthreads();
    uint32_t before = 0;
#pragma unroll
    for (int w = 0; w < kRegWaves; ++w)
        if (w < wave) before += wave_tot[w];
    int G = static_cast<int>(before & 0xffffu), Q = static_cast<int>(before >> 16);   // keys before this round
    // T read back from LDS, so that the compares are redone here rather than
    // kept from the count above (64 keys' masks would not fit in SGPRs); the
    // ids likewise are computed afresh from an opaque copy of `base` (kept
    // from the loads, their 16 registers would push keys out to scratch)
    const uint32_t T2 = s_T;
    int base2 = base;
    asm volatile("" : "+v"(base2));
    // keys of this lane's lower-numbered lanes
    const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
    for (int r = 0; r < kRegRounds; ++r) {
        // ranks inside the round from ballots of the lanes' keys above and
        // equal to T: a kept key's place is the round's kept keys in lower
        // lanes, then this lane's earlier keys
        uint64_t mg[4], mq[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            mg[c] = __builtin_amdgcn_ballot_w64(rk[4 * r + c] > T2);
            mq[c] = __builtin_amdgcn_ballot_w64(rk[4 * r + c] == T2);
        }
        int gb = G, qb = Q;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            gb += __builtin_popcountll(mg[c] & below);
            qb += __builtin_popcountll(mq[c] & below);
            G += __builtin_popcountll(mg[c]);
            Q += __builtin_popcountll(mq[c]);
        }
        const int j = base2 + 256 * r;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint32_t key = rk[4 * r + c];
            const bool gt = key > T2, eq = key == T2;
            const int slot = gt ? gb + min(qb, remaining) : (eq && qb < remaining) ? gb + qb : kTopKMax + lane;
            ostage[slot] = j + c;
            gb += gt;
            qb += eq;
        }
    }
    __syncthreads();
    for (int k = tid; k < top_k; k += kRegThreads) out[k] = ostage[k];
    if (tid == 0) n_sel[i] = top_k;
}

// ---------------------------------------------------------------------------
// Few queries over more than one chunk of keys: the same selection spread
// over one workgroup per 8192-key chunk, so that a 16-query call over 64K
// keys keeps 128 compute units busy instead of 16.
//  1. dsa_chunk_hist_kernel: each chunk's histogram of the top 12 key bits
//     (u16 counts) into the workspace.
//  2. dsa_chunk_split_kernel: each chunk's workgroup adds up its query's
//     chunk histograms, picks the boundary digit d1 as the one-workgroup
//     kernels do, and writes the ids of its keys above the boundary bin (all
//     of them kept) and the keys and ids of those inside it, each list at the
//     offset the earlier chunks' counts give, so both are in id order.
//  3. dsa_finish_kernel: one workgroup per query resolves the last 12 + 8
//     bits over the boundary list (copied into LDS when it fits), marks the
//     above-bin ids, the boundary keys > T and the lowest-id keys == T in a
//     bit map of the ids, and writes the marked ids in order (each thread's
//     place from a scan of its map words' popcounts).
// ---------------------------------------------------------------------------
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
constexpr int kChunk = 8192;
constexpr int kMwThreads = 1024;
constexpr int kMwPer = kChunk / kMwThreads;             // 8 consecutive keys per thread
constexpr int kMwMaxQueries = 32;
constexpr int kMwMaxChunks = kRegKeys / kChunk;         // 8
constexpr int kMwHistCopies = 4;
constexpr int kFinCap = 8192;                           // boundary entries the finishing kernel holds in LDS

bool use_chunks(int64_t n_q, int32_t max_pos) {
    const int64_t n = static_cast<int64_t>(max_pos) + 1;
    return n_q <= kMwMaxQueries && n > kChunk && n <= kRegKeys;
}
int n_chunks_of(int32_t max_pos) { return (max_pos + kChunk) / kChunk; }

// Workspace after the scores: chunk histograms [n_q][n_chunks][4096] u16 |
// {d1, keys still needed from bin d1, above count, boundary count} [n_q] |
// above-bin ids [n_q][4096] | boundary keys [n_q][stride] | boundary ids
// [n_q][stride], each region 256-byte aligned.
struct ChunkLayout {
    size_t hist, meta, above, bkey, bid, total;
};

__global__ __launch_bounds__(kMwThreads) void dsa_chunk_hist_kernel(const float* __restrict__ scores, int64_t stride,
                                                                    const int32_t* __restrict__ q_pos, int top_k,
                                                                    int n_chunks, uint16_t* __restrict__ hist_g) {
    __shared__ int hist[kMwHistCopies][kBins];
    const int w = blockIdx.x;
    const int64_t i = blockIdx.y;
    const int tid = threadIdx.x;
    const int n = min(q_pos[i] + 1, static_cast<int>(stride));   // (positions lie in the rows)
    const int c0 = w * kChunk;
    if (n <= top_k || c0 >= n) return;                  // workgroup-uniform
    const float* t = scores + i * stride;
    // keys j0 .. j0 + 7 (a thread whose keys all lie past the row's end
    // reads the row's last eight scores instead, and counts none)
    const int j0 = c0 + kMwPer * tid;
    const int jl = min(j0, static_cast<int>(stride) - kMwPer);
    const f32x4 x0 = *reinterpret_cast<const f32x4*>(t + jl);
    const f32x4 x1 = *reinterpret_cast<const f32x4*>(t + jl + 4);
    for (int b = tid; b < kMwHistCopies * kBins; b += kMwThreads) (&hist[0][0])[b] = 0;
    __syncthreads();
    const float xs[kMwPer] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    int* hc = hist[tid % kMwHistCopies];
#pragma unroll
    for (int e = 0; e < kMwPer; ++e)
        if (j0 + e < n) atomicAdd(&hc[ordered_key(xs[e]) >> 20], 1);
    __syncthreads();
    // thread t: bins 4t .. 4t + 3 (at most 8192 keys each: u16)
    uint32_t c[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        int sum = 0;
#pragma unroll
        for (int k = 0; k < kMwHistCopies; ++k) sum += hist[k][4 * tid + b];
        c[b] = static_cast<uint32_t>(sum);
    }
    *reinterpret_cast<u32x2*>(hist_g + ((i * n_chunks + w) * kBins + 4 * tid)) = u32x2{c[0] | (c[1] << 16), c[2] | (c[3] << 16)};
}

struct SplitArgs {
    const float* scores;
    int64_t stride;
    const int32_t* q_pos;
    int top_k;
    int n_chunks;
    const uint16_t* hist;
    int32_t* meta;
    int32_t* above;
    uint32_t* bkey;
    int32_t* bid;
};

__global__ __launch_bounds__(kMwThreads) void dsa_chunk_split_kernel(SplitArgs a) {
    __shared__ int hist[kBins];
    __shared__ int wave_sums[kMwThreads / 64];
    __shared__ uint32_t s_digit;
    __shared__ int s_remaining;
    __shared__ int s_above[kMwMaxChunks];
    __shared__ int s_inbin[kMwMaxChunks];
    const int w = blockIdx.x;
    const int64_t i = blockIdx.y;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int n = min(a.q_pos[i] + 1, static_cast<int>(a.stride));
    const int nch = (n + kChunk - 1) / kChunk;
    if (n <= a.top_k || w >= nch) return;               // workgroup-uniform
    if (tid < kMwMaxChunks) {
        s_above[tid] = 0;
        s_inbin[tid] = 0;
    }
    // bins 4t .. 4t + 3 of every chunk histogram of the query (chunks past
    // the query's last key re-read its last chunk and count as empty), then
    // the thread's own eight keys, all loads in flight together
    u32x2 hc[kMwMaxChunks];
#pragma unroll
    for (int k = 0; k < kMwMaxChunks; ++k) {
        const int kk = min(k, nch - 1);
        hc[k] = *reinterpret_cast<const u32x2*>(a.hist + ((i * a.n_chunks + kk) * kBins + 4 * tid));
    }
    const float* t = a.scores + i * a.stride;
    const int j0 = w * kChunk + kMwPer * tid;
    const int jl = min(j0, static_cast<int>(a.stride) - kMwPer);
    const f32x4 x0 = *reinterpret_cast<const f32x4*>(t + jl);
    const f32x4 x1 = *reinterpret_cast<const f32x4*>(t + jl + 4);
    auto count = [&](int k, int b) __attribute__((always_inline)) {
        const uint32_t word = (b & 2) ? hc[k].y : hc[k].x;
        return k < nch ? static_cast<int>((word >> (16 * (b & 1))) & 0xffffu) : 0;
    };
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        int sum = 0;
#pragma unroll
        for (int k = 0; k < kMwMaxChunks; ++k) sum += count(k, b);
        hist[4 * tid + b] = sum;
    }
    __syncthreads();
    pick_digit_t<kMwThreads>(hist, 12, a.top_k, wave_sums, &s_digit, &s_remaining);
    const int d1 = static_cast<int>(s_digit);
    const int r1 = s_remaining;
    // per chunk: keys above bin d1 (a sum over the workgroup; two chunks'
    // counts share an int, at most 8192 each) and in it (one thread holds
    // that bin)
#pragma unroll
    for (int k = 0; k < kMwMaxChunks; k += 2) {
        int av = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) av += 4 * tid + b > d1 ? count(k, b) + (count(k + 1, b) << 16) : 0;
        av = wave_sum(av);
        if (lane == 0 && av) {
            atomicAdd(&s_above[k], av & 0xffff);
            atomicAdd(&s_above[k + 1], av >> 16);
        }
    }
    if ((d1 >> 2) == tid) {
#pragma unroll
        for (int k = 0; k < kMwMaxChunks; ++k) s_inbin[k] = count(k, d1 & 3);
    }
    __syncthreads();
    int A = 0, B = 0, NA = 0, NB = 0;
#pragma unroll
    for (int k = 0; k < kMwMaxChunks; ++k) {
        if (k < w) {
            A += s_above[k];
            B += s_inbin[k];
        }
        NA += s_above[k];
        NB += s_inbin[k];
    }
    const float xs[kMwPer] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    uint32_t key[kMwPer];
    int na_t = 0, nb_t = 0;
#pragma unroll
    for (int e = 0; e < kMwPer; ++e) {
        key[e] = ordered_key(xs[e]);
        const bool valid = j0 + e < n;
        const int dig = static_cast<int>(key[e] >> 20);
        na_t += valid && dig > d1;
        nb_t += valid && dig == d1;
    }
    // (at most 8192 keys per chunk: the two counts share one int)
    const int packed = na_t + (nb_t << 16);
    const int excl = block_scan<kMwThreads>(packed, wave_sums) - packed;
    int oa = A + (excl & 0xffff), ob = B + (excl >> 16);
    int32_t* above = a.above + i * kTopKMax;
    uint32_t* bkey = a.bkey + i * a.stride;
    int32_t* bid = a.bid + i * a.stride;
#pragma unroll
    for (int e = 0; e < kMwPer; ++e) {
        if (j0 + e < n) {
            const int dig = static_cast<int>(key[e] >> 20);
            // (the bounds hold by the counts; kept as guards)
            if (dig > d1) {
                if (oa < kTopKMax) above[oa] = j0 + e;
                ++oa;
            } else if (dig == d1) {
                if (ob < n) {
                    bkey[ob] = key[e];
                    bid[ob] = j0 + e;
                }
                ++ob;
            }
        }
    }
    if (w == 0 && tid == 0) *reinterpret_cast<int4*>(a.meta + 4 * i) = make_int4(d1, r1, NA, NB);
}

struct FinishArgs {
    const int32_t* q_pos;
    int top_k;
    int64_t stride;
    const int32_t* meta;
    const int32_t* above;
    const uint32_t* bkey;
    const int32_t* bid;
    int32_t* sel;
    int32_t* n_sel;
};

__global__ __launch_bounds__(kMwThreads) void dsa_finish_kernel(FinishArgs a) {
    __shared__ int hist[kBins];
    __shared__ uint32_t lkey[kFinCap];
    __shared__ int32_t lid[kFinCap];
    __shared__ uint32_t idmap[kRegKeys / 32];           // kept ids, one bit each
    __shared__ int wave_sums[kMwThreads / 64];
    __shared__ uint32_t s_digit;
    __shared__ int s_remaining;
    const int64_t i = blockIdx.x;
    const int tid = threadIdx.x;
    const int n = min(a.q_pos[i] + 1, static_cast<int>(a.stride));
    const int top_k = a.top_k;
    int32_t* out = a.sel + i * top_k;
    if (n <= top_k) {                                   // every visible key is kept
        for (int j = tid; j < top_k; j += kMwThreads) out[j] = j < n ? j : -1;
        if (tid == 0) a.n_sel[i] = n;
        return;
    }
    // the counts, the first kSpec list entries and the above-bin ids (fewer
    // than top_k) are loaded together, before the counts are known (the
    // lists hold at least 8192 and kTopKMax entries: a row of more than 8192
    // scores each); a longer list that fits in LDS takes a second round
    const int4 m = *reinterpret_cast<const int4*>(a.meta + 4 * i);
    const uint32_t* gkey = a.bkey + i * a.stride;
    const int32_t* gid = a.bid + i * a.stride;
    constexpr int kSpec = 2048;
    constexpr int kLd = kSpec / kMwThreads, kLa = kTopKMax / kMwThreads;
    uint32_t kk[kLd];
    int32_t ii[kLd], aa[kLa];
#pragma unroll
    for (int r = 0; r < kLd; ++r) {
        kk[r] = gkey[tid + kMwThreads * r];
        ii[r] = gid[tid + kMwThreads * r];
    }
#pragma unroll
    for (int r = 0; r < kLa; ++r) {
        const int e = tid + kMwThreads * r;
        aa[r] = e < top_k ? a.above[i * kTopKMax + e] : 0;
    }
    for (int wd = tid; wd < kRegKeys / 32; wd += kMwThreads) idmap[wd] = 0u;
    const int d1 = m.x, na = m.z, nb = m.w;
    const bool in_lds = nb <= kFinCap;                   // workgroup-uniform
#pragma unroll
    for (int r = 0; r < kLd; ++r) {
        lkey[tid + kMwThreads * r] = kk[r];
        lid[tid + kMwThreads * r] = ii[r];
    }
    if (in_lds) {
        for (int e = kSpec + tid; e < nb; e += kMwThreads) {
            lkey[e] = gkey[e];
            lid[e] = gid[e];
        }
    }
    const uint32_t* keys = in_lds ? lkey : gkey;
    const int32_t* ids = in_lds ? lid : gid;
    uint32_t prefix = static_cast<uint32_t>(d1) << 20, mask = 0xfff00000u;
    int remaining = m.y;
#pragma unroll
    for (int pass = 1; pass < 3; ++pass) {
        const int bits = kDigitBits[pass];
        const int shift = pass == 1 ? 8 : 0;
        const uint32_t dmask = (1u << bits) - 1;
        for (int b = tid; b < kBins; b += kMwThreads) hist[b] = 0;
        __syncthreads();
        for (int e = tid; e < nb; e += kMwThreads) {
            const uint32_t key = keys[e];
            if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1);
        }
        __syncthreads();
        pick_digit_t<kMwThreads>(hist, bits, remaining, wave_sums, &s_digit, &s_remaining);
        prefix |= s_digit << shift;
        mask |= dmask << shift;
        remaining = s_remaining;
    }
    const uint32_t T = prefix;          // the top_k-th largest key; `remaining` boundary keys equal to it are kept
    // kept ids into the bit map: every above-bin id, the boundary keys > T
    // and the first `remaining` boundary keys == T in list (= id) order
    // (thread t takes entries [t * per, (t + 1) * per))
    auto keep = [&](int32_t id) __attribute__((always_inline)) {
        atomicOr(&idmap[(id >> 5) & (kRegKeys / 32 - 1)], 1u << (id & 31));
    };
#pragma unroll
    for (int r = 0; r < kLa; ++r)
        if (tid + kMwThreads * r < na) keep(aa[r]);
    const int per = (nb + kMwThreads - 1) / kMwThreads;
    const int e0 = min(tid * per, nb), e1 = min(e0 + per, nb);
    int n_eq = 0;
    for (int e = e0; e < e1; ++e) n_eq += keys[e] == T;
    int eq_rank = block_scan<kMwThreads>(n_eq, wave_sums) - n_eq;
    for (int e = e0; e < e1; ++e) {
        const uint32_t key = keys[e];
        if (key > T) {
            keep(ids[e]);
        } else if (key == T) {
            if (eq_rank < remaining) keep(ids[e]);
            ++eq_rank;
        }
    }
    __syncthreads();
    // the output in id order: thread t writes the kept ids of its two words
    // (ids 64t .. 64t + 63) after the kept ids of the lower words
    const uint32_t w0 = idmap[2 * tid], w1 = idmap[2 * tid + 1];
    const int c = __builtin_popcount(w0) + __builtin_popcount(w1);
    int o = block_scan<kMwThreads>(c, wave_sums) - c;
    uint64_t bm = static_cast<uint64_t>(w0) | (static_cast<uint64_t>(w1) << 32);
    while (bm) {
        const int b = __builtin_ctzll(bm);
        if (o < top_k) out[o] = 64 * tid + b;           // exactly top_k bits are set; the bound is defensive
        ++o;
        bm &= bm - 1;
    }
    if (tid == 0) a.n_sel[i] = top_k;
}

int64_t score_stride(int32_t max_pos) {
    return ((static_cast<int64_t>(max_pos) + 1 + 63) / 64) * 64;
}

ChunkLayout chunk_layout(int64_t n_q, int32_t max_pos) {
    const size_t stride = static_cast<size_t>(score_stride(max_pos));
    auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
    ChunkLayout l;
    l.hist = up(static_cast<size_t>(n_q) * stride * sizeof(float));
    l.meta = l.hist + up(static_cast<size_t>(n_q) * n_chunks_of(max_pos) * kBins * sizeof(uint16_t));
    l.above = l.meta + up(static_cast<size_t>(n_q) * 4 * sizeof(int32_t));
    l.bkey = l.above + up(static_cast<size_t>(n_q) * kTopKMax * sizeof(int32_t));
    l.bid = l.bkey + up(static_cast<size_t>(n_q) * stride * sizeof(uint32_t));
    l.total = l.bid + static_cast<size_t>(n_q) * stride * sizeof(int32_t);
    return l;
}

hipError_t launch_topk(void* ws, int64_t stride, const int32_t* pos, int64_t n_q, int32_t max_pos,
                       int top_k, int32_t* sel, int32_t* n_sel, hipStream_t s) {
    const float* scores = static_cast<const float*>(ws);
    if (use_chunks(n_q, max_pos)) {
        const ChunkLayout l = chunk_layout(n_q, max_pos);
        char* base = static_cast<char*>(ws);
        const int nc = n_chunks_of(max_pos);
        uint16_t* hist = reinterpret_cast<uint16_t*>(base + l.hist);
        int32_t* meta = reinterpret_cast<int32_t*>(base + l.meta);
        int32_t* above = reinterpret_cast<int32_t*>(base + l.above);
        uint32_t* bkey = reinterpret_cast<uint32_t*>(base + l.bkey);
        int32_t* bid = reinterpret_cast<int32_t*>(base + l.bid);
        const dim3 grid(static_cast<unsigned>(nc), static_cast<unsigned>(n_q));
        hipLaunchKernelGGL(dsa_chunk_hist_kernel, grid, dim3(kMwThreads), 0, s, scores, stride, pos, top_k, nc, hist);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(dsa_chunk_split_kernel, grid, dim3(kMwThreads), 0, s,
                           SplitArgs{scores, stride, pos, top_k, nc, hist, meta, above, bkey, bid});
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(dsa_finish_kernel, dim3(static_cast<unsigned>(n_q)), dim3(kMwThreads), 0, s,
                           FinishArgs{pos, top_k, stride, meta, above, bkey, bid, sel, n_sel});
        return hipGetLastError();
    }
    if (static_cast<int64_t>(max_pos) + 1 <= kRegKeys)
        hipLaunchKernelGGL(dsa_topk_regs_kernel, dim3(static_cast<unsigned>(n_q)), dim3(kRegThreads), 0, s, scores,
                           stride, pos, top_k, sel, n_sel);
    else
        hipLaunchKernelGGL(dsa_topk_kernel, dim3(static_cast<unsigned>(n_q)), dim3(kSelThreads), 0, s, scores,
                           stride, pos, top_k, sel, n_sel);
    return hipGetLastError();
}

}  // namespace

size_t dsa_select_ws_bytes(int64_t n_q, int32_t max_pos) {
    if (use_chunks(n_q, max_pos)) return chunk_layout(n_q, max_pos).total;
    return static_cast<size_t>(n_q) * score_stride(max_pos) * sizeof(float);
}

hipError_t launch_dsa_select(const uint16_t* dsa_k, const Pager& pg, const uint16_t* q_idx,
                             const int32_t* stream, const int32_t* pos, int64_t n_q,
                             int32_t max_pos, int top_k, int32_t* sel, int32_t* n_sel, void* ws,
                             hipStream_t s) {
    float* scores = static_cast<float*>(ws);
    const int64_t stride = score_stride(max_pos);
    const unsigned nx = static_cast<unsigned>((max_pos + kScoreKeysPerWg) / kScoreKeysPerWg);
    hipLaunchKernelGGL(dsa_score_kernel, dim3(nx, static_cast<unsigned>(n_q)), dim3(256), 0, s, dsa_k,
                       pg, q_idx, stream, pos, scores, stride);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_topk(ws, stride, pos, n_q, max_pos, top_k, sel, n_sel, s);
}

hipError_t launch_dsa_select_heads(const uint16_t* dsa_k, const Pager& pg, const uint16_t* q_idx_h,
                                   const float* head_w, int n_head, const int32_t* stream,
                                   const int32_t* pos, int64_t n_q, int32_t max_pos, int top_k,
                                   int32_t* sel, int32_t* n_sel, void* ws, hipStream_t s) {
    float* scores = static_cast<float*>(ws);
    const int64_t stride = score_stride(max_pos);
    const dim3 grid(static_cast<unsigned>((max_pos + kMhKeysPerWg) / kMhKeysPerWg), static_cast<unsigned>(n_q));
    const dim3 block(64 * kMhWaves);
    switch (n_head) {
        case 16: hipLaunchKernelGGL(dsa_score_heads_kernel<1>, grid, block, 0, s, dsa_k, pg, q_idx_h, head_w,
                                    stream, pos, scores, stride); break;
        case 32: hipLaunchKernelGGL(dsa_score_heads_kernel<2>, grid, block, 0, s, dsa_k, pg, q_idx_h, head_w,
                                    stream, pos, scores, stride); break;
        case 48: hipLaunchKernelGGL(dsa_score_heads_kernel<3>, grid, block, 0, s, dsa_k, pg, q_idx_h, head_w,
                                    stream, pos, scores, stride); break;
        case 64: hipLaunchKernelGGL(dsa_score_heads_kernel<4>, grid, block, 0, s, dsa_k, pg, q_idx_h, head_w,
                                    stream, pos, scores, stride); break;
        default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_topk(ws, stride, pos, n_q, max_pos, top_k, sel, n_sel, s);
}

}  // namespace msa
