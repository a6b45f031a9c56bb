// prefill_attend.hip -- block-sparse attention for a prefill chunk.
//
// "Add MiniMax-M3 (MSA: MiniMax Sparse Attention) support", Implementation,
// batch path: each query attends only over its group's selected blocks
// (causal inside the query's own block); prefill and decode rank the same
// block scores, so the selection semantics are those of decode.
//
// Design (gfx950).  A workgroup owns a tile of 32 consecutive queries of one
// group and sweeps the union of their selected blocks in ascending block
// order, so each block's K and V are fetched once per tile (and, since every
// workgroup of an XCD sweeps the same group upward at the same time, mostly
// from that XCD's L2).  A small pre-kernel turns the selections into each
// tile's step list: one step per union block and up to kPb of the tile's
// queries that selected it (a block chosen by more queries, e.g. the shared
// local block, becomes several steps).
//
// Every step is spread evenly over all eight waves, whatever queries it
// holds: for S = Q K^T wave w takes keys 16w .. 16w+15 of the block for every
// query of the step and writes its bf16 probabilities to LDS; for O += P V
// wave w owns output dims 16w .. 16w+15 of all 32 queries of the tile, so the
// 16-head x 128-dim accumulators of the whole tile live in registers, one
// 16 x 16 slice per wave and query.  The softmax needs no exchange of maxima:
// each (query, head) uses one fixed reference for the whole sweep (its score
// against its own key, always selected), and a block whose probabilities
// would pass 2^64 is recomputed against a raised reference (rare).  The
// owner wave of each query sums the bf16 probabilities it reads as P V
// operands (v_dot2 against ones), so the normalisation sums exactly the
// weights applied.
//
// The sweep is pipelined by one step with a single barrier per step: the
// interval between barriers i - 1 and i holds the scores of step i and the
// products P V of step i - 1, with probabilities, V and the step's queries
// in two-deep LDS rings (K goes straight from memory into the registers of
// the wave that uses it and never passes through LDS).  During the interval
// the copies for the next interval are issued, spread over its phases (step
// i + 1's queries as it begins, half of step i's V, then step i + 1's K and
// the other half of V once the scores are done): the copy engine accepts
// about 49 bytes per clock per compute unit, so copies issued all at once
// stall every wave until they drain.
#include "common.hpp"

namespace msa {
namespace {

constexpr int kPaWaves = 8;
constexpr int kPaThreads = 64 * kPaWaves;
constexpr int kTq = 32;                     // queries per tile (one mask bit each)
constexpr int kPb = 5;                      // queries per step
constexpr int kRowBytes = kHeadDim * 2;     // one group's K or V row, one head's Q row: 256 B
constexpr int kBufBytes = kBlock * kRowBytes;        // 32 KiB: K (or V) of one block
constexpr int kQBytes = kHeadsPerGroup * kRowBytes;  // 4 KiB: one query's 16 heads
constexpr float kLog2eP = 1.4426950408889634f;
constexpr int kStepsThreads = 256;

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

// Rows are stored with their 16 segments permuted by seg ^ f(row & 15), f a
// 4-bit rotate: f is one-to-one on 16 consecutive rows (operand reads of 16
// rows at one segment) and f >> 1 is one-to-one on 8 consecutive rows (the
// transposing V reads take a 32-byte pair of segments from each of 8 rows per
// half-wave), so neither read pattern has bank conflicts.
__device__ __forceinline__ int rowperm(int row) { return ((row & 7) << 1) | ((row >> 3) & 1); }
// Byte offset of 16-byte segment `seg` of row `row` in a staged buffer.
__device__ __forceinline__ int swz(int row, int seg) { return row * kRowBytes + ((seg ^ rowperm(row)) << 4); }

// Workgroup barrier that orders LDS accesses only: this wave's LDS reads and
// writes complete (lgkmcnt 0) before it arrives, while copies into LDS still
// in flight (global_load_lds, counted by vmcnt) are not waited for.  The
// empty asm statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);        // vmcnt 63, expcnt 7, lgkmcnt 0
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), bf16x2_t));
}

// ---------------------------------------------------------------------------
// Step lists.  Workgroup (tile, g): entry = {block id, mask of tile queries,
// first cache row of the block (low, high word)}, ascending block order, at
// most kPb mask bits per entry.  The row is resolved here, through the block
// table of a paged cache, so that the sweep does no table lookups.
// ---------------------------------------------------------------------------
struct StepArgs {
    const int32_t* sel;
    int top_k;
    int pos0;
    int64_t n_q;
    int nblk;
    int max_steps;
    Pager pg;
    int32_t stream;
    int32_t* counts;
    u32x4* steps;
};

__global__ __launch_bounds__(kStepsThreads) void prefill_steps_kernel(StepArgs a) {
    const int g = blockIdx.x % kGroups;
    const int64_t q_first = static_cast<int64_t>(blockIdx.x / kGroups) * kTq;
    const int n_tq = static_cast<int>(min<int64_t>(kTq, a.n_q - q_first));
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    extern __shared__ uint32_t qmask[];        // [nblk]
    __shared__ int wave_sums[kStepsThreads / 64];

    for (int b = threadIdx.x; b < a.nblk; b += kStepsThreads) qmask[b] = 0u;
    __syncthreads();
    for (int e = threadIdx.x; e < n_tq * a.top_k; e += kStepsThreads) {
        const int t = e / a.top_k;
        const int64_t qi = q_first + t;
        const int blk = a.sel[(qi * kGroups + g) * a.top_k + e % a.top_k];
        const int loc = (a.pos0 + static_cast<int>(qi)) / kBlock;
        if (blk >= 0 && blk <= loc) atomicOr(&qmask[blk], 1u << t);
    }
    __syncthreads();
    // steps per block, exclusive scan over the workgroup in block order
    const int per = (a.nblk + kStepsThreads - 1) / kStepsThreads;
    const int b0 = threadIdx.x * per, b1 = min(b0 + per, a.nblk);
    int cnt = 0;
    for (int b = b0; b < b1; ++b) cnt += (__builtin_popcount(qmask[b]) + kPb - 1) / kPb;
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
    }
    if (lane == 63) wave_sums[wave] = incl;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += wave_sums[w];
    int pos = before + incl - cnt;
    u32x4* out = a.steps + static_cast<int64_t>(blockIdx.x) * a.max_steps;
    for (int b = b0; b < b1; ++b) {
        uint32_t m = qmask[b];
        const uint64_t row = m != 0u ? static_cast<uint64_t>(a.pg.block_row(a.stream, b)) : 0u;
        while (m != 0u) {
            uint32_t sub = 0u;
            for (int i = 0; i < kPb && m != 0u; ++i) {
                const uint32_t low = m & (~m + 1u);
                sub |= low;
                m ^= low;
            }
            out[pos++] = u32x4{static_cast<uint32_t>(b), sub, static_cast<uint32_t>(row),
                               static_cast<uint32_t>(row >> 32)};
        }
    }
    if (threadIdx.x == kStepsThreads - 1) a.counts[blockIdx.x] = before + incl;
}

// ---------------------------------------------------------------------------
// Attention sweep.
// ---------------------------------------------------------------------------
struct PaArgs {
    const uint16_t* k;
    const uint16_t* v;
    Pager pg;
    const uint16_t* q;
    int32_t stream;
    int32_t pos0;
    int64_t n_q;
    int64_t last_row;
    int max_steps;
    const int32_t* counts;
    const u32x4* steps;
    float scale;
    float* out;
};

__global__ __launch_bounds__(kPaThreads, 1) void prefill_attend_kernel(PaArgs a) {
    const int g = blockIdx.x % kGroups;
    const int64_t q_first = static_cast<int64_t>(blockIdx.x / kGroups) * kTq;
    const int n_tq = a.n_q - q_first < kTq ? static_cast<int>(a.n_q - q_first) : kTq;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l16 = lane & 15;
    const int l4 = lane >> 4;
    const int n_steps = a.counts[blockIdx.x];
    const u32x4* steps = a.steps + static_cast<int64_t>(blockIdx.x) * a.max_steps;
    // the same list read through the scalar cache (entries are wave-uniform)
    const __attribute__((address_space(4))) u32x4* steps_s =
        (const __attribute__((address_space(4))) u32x4*)(reinterpret_cast<uintptr_t>(steps));

    // Two-deep rings (by step parity) for V, the step's queries and its
    // probabilities.  Separate objects, so that reads of one are not made to
    // wait for copies in flight into another.  K does not pass through LDS:
    // each wave loads its own 16 keys straight into the registers the score
    // products read.
    __shared__ __attribute__((aligned(16))) char vbuf0[kBufBytes];
    __shared__ __attribute__((aligned(16))) char vbuf1[kBufBytes];
    __shared__ __attribute__((aligned(16))) char qbuf0[kPb][kQBytes];
    __shared__ __attribute__((aligned(16))) char qbuf1[kPb][kQBytes];
    __shared__ __attribute__((aligned(16))) char pbuf0[kPb][kQBytes];
    __shared__ __attribute__((aligned(16))) char pbuf1[kPb][kQBytes];
    __shared__ __attribute__((aligned(16))) float pmax[kPb][kHeadsPerGroup][kPaWaves];
    __shared__ float rnew[kPb][kHeadsPerGroup];    // redo: raised reference of the step's queries
    __shared__ float alph[kPb][kHeadsPerGroup];    // redo: accumulator factor
    __shared__ float m_ref[kTq][kHeadsPerGroup];   // reference of each (query, head), log2 units
    __shared__ float l_fin[kTq][kHeadsPerGroup];
    __shared__ int redo_step[2];                   // last step of each parity whose probabilities overflowed

    const float qk_scale = a.scale * kLog2eP;
    const int64_t q_base = (q_first * kGroups + g) * kHeadsPerGroup * kHeadDim;   // query q_first's 16 heads
    constexpr int64_t kQStride = int64_t(kGroups) * kHeadsPerGroup * kHeadDim;     // next query

    // Softmax reference of (query t, head h): its score against its own key,
    // which every selection holds (the local block is always selected).  Any
    // finite reference gives the same softmax; this one keeps the query's
    // largest probability at or above 1, and a block whose probabilities
    // would pass 2^kOverflow raises it (the step is redone, see below).
    {
        const int t = threadIdx.x >> 4, h = threadIdx.x & 15;
        float r = 0.f;
        if (t < n_tq) {
            const uint16_t* qr = a.q + q_base + t * kQStride + h * kHeadDim;
            const uint16_t* kr = a.k + (a.pg.row(a.stream, a.pos0 + static_cast<int>(q_first) + t) * kGroups + g) * kHeadDim;
            float s0 = 0.f, s1 = 0.f;
#pragma unroll 4
            for (int d = 0; d < kHeadDim; d += 8) {
                const u32x4 qa = *reinterpret_cast<const u32x4*>(qr + d);
                const u32x4 ka = *reinterpret_cast<const u32x4*>(kr + d);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    s0 = __builtin_fmaf(__uint_as_float(qa[j] << 16), __uint_as_float(ka[j] << 16), s0);
                    s1 = __builtin_fmaf(__uint_as_float(qa[j] & 0xffff0000u), __uint_as_float(ka[j] & 0xffff0000u), s1);
                }
            }
            r = (s0 + s1) * qk_scale;
        }
        m_ref[t][h] = r;
        if (threadIdx.x < 2) redo_step[threadIdx.x] = -1;
    }
    // O^T slices (dims 16w + 4*l4 + r, head l16) of all tile queries, and
    // the row sums of the queries t with t % 8 == w: lane (l16, l4) sums the
    // bf16 probabilities of head l16 it reads as operands (keys 32c + 8*l4
    // .. +7), so that the normalisation sums exactly the weights applied
    f32x4 acc[kTq];
    float lsum[kTq / kPaWaves];
#pragma unroll
    for (int t = 0; t < kTq; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < kTq / kPaWaves; ++k) lsum[k] = 0.f;

    // Lane offsets inside staged buffers (the row permutation depends on
    // row & 15 only, so multiples of 16 rows are added as constants).
    int qoff[4];                                // Q rows (heads) l16, dims 32*ks4 + 8*l4 ..
#pragma unroll
    for (int ks4 = 0; ks4 < 4; ++ks4) qoff[ks4] = swz(l16, 4 * ks4 + l4);
    // V: row 4*l4 + l16/4 (+ 32c, + 16), dims 16w + 4*(l16 % 4) .. +3
    const int voff = swz(4 * l4 + (l16 >> 2), 2 * wave + ((l16 & 3) >> 1)) + (l16 & 1) * 8;
    // P exchange: chunk c = keys 32c .. 32c+31 is written by waves 2c (keys
    // 32c + 4*l4 + r) and 2c+1 (keys 32c + 16 + 4*l4 + r) and read as the
    // 8-key B operand of lane (l16, l4) of every wave.
    const int pw_off = (((wave >> 1) * 4 + l4) * 16 + l16) * 16 + (wave & 1) * 8;
    const int pr_off = (l4 * 16 + l16) * 16;   // + 1 KiB per chunk

    // Copies of V.  Slot s (16 bytes) of a staged 256-byte-row buffer holds
    // segment (s % 16) ^ f(row) of row s / 16.  One call issues instruction j
    // (of 4) of this wave's share of the block.
    const int last_row = static_cast<int>(a.last_row);       // positions are int32
    uint32_t soff[4];                                          // lane's source offset (elements) in a block
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int slot = 256 * wave + 64 * j + lane;
        const int row = slot >> 4;
        soff[j] = static_cast<uint32_t>(row * kGroups * kHeadDim + 8 * ((slot & 15) ^ rowperm(row)));
    }
    // e: the block's step entry (block id, mask, first cache row)
    auto stage_v = [&](const u32x4& e, char* dst, int j) {
        const int row0 = static_cast<int>(e[0]) * kBlock;
        const int64_t rb = static_cast<int64_t>((static_cast<uint64_t>(e[3]) << 32) | e[2]);
        const uint16_t* src = a.v + (rb * kGroups + g) * kHeadDim;
        uint32_t o = soff[j];
        if (row0 + kBlock - 1 > last_row) {                   // wave-uniform: the chunk's last block
            // rows past the chunk's last key are read from that key's row:
            // they are masked for every query
            const int row = (256 * wave + 64 * j + lane) >> 4;
            o -= static_cast<uint32_t>((row - min(row, last_row - row0)) * kGroups * kHeadDim);
        }
        __builtin_amdgcn_global_load_lds(src + o, LDS_PTR(void, dst + (256 * wave + 64 * j) * 16), 16, 0, 0);
    };
    // K of this wave's keys 16w + l16 into registers: lane (l16, l4) holds
    // dims 32*ks4 + 8*l4 .. +7 in kr[ks4], the A operand of the score products.
    auto load_k = [&](const u32x4& e, bf16x8 (&kr)[4]) {
        const int row0 = static_cast<int>(e[0]) * kBlock;
        const int64_t rb = static_cast<int64_t>((static_cast<uint64_t>(e[3]) << 32) | e[2]);
        int row = 16 * wave + l16;
        if (row0 + kBlock - 1 > last_row) row = min(row, last_row - row0);   // past the chunk's last key: masked
        const uint16_t* src = a.k + ((rb + row) * kGroups + g) * kHeadDim + 8 * l4;
#pragma unroll
        for (int ks4 = 0; ks4 < 4; ++ks4) kr[ks4] = *reinterpret_cast<const bf16x8*>(src + 32 * ks4);
    };
    // Q of query t into slot p of qdst: instruction j (of 4) is issued by wave (4p + j) % 8.
    auto stage_q = [&](char (*qdst)[kQBytes], int p, int t) {
        const int j = (wave - 4 * p) & 7;
        if (j < 4) {
            const int slot = 64 * j + lane;
            const int row = slot >> 4;
            const int seg = (slot & 15) ^ rowperm(row);
            __builtin_amdgcn_global_load_lds(a.q + q_base + t * kQStride + row * kHeadDim + 8 * seg,
                                             LDS_PTR(void, &qdst[p][64 * j * 16]), 16, 0, 0);
        }
    };
    // (unrolled over the slots, so that every copy's LDS destination is a
    // known object and reads of other buffers need not wait for it)
    auto stage_queries = [&](const u32x4& e, char (*qdst)[kQBytes]) {
        uint32_t m = e[1];
#pragma unroll
        for (int p = 0; p < kPb; ++p) {
            if (m != 0u) {
                stage_q(qdst, p, __builtin_ctz(m));
                m &= m - 1u;
            }
        }
    };

    // This wave's S^T tile (keys 16w + 4*l4 + r, head l16) of query p of the
    // step, from K in registers and Q in qs[p]; keys past the query masked.
    auto load_q = [&](const char (*qs)[kQBytes], int p, bf16x8 (&qop)[4]) {
#pragma unroll
        for (int ks4 = 0; ks4 < 4; ++ks4) qop[ks4] = *reinterpret_cast<const bf16x8*>(qs[p] + qoff[ks4]);
    };
    auto score_q = [&](const bf16x8 (&kop)[4], const bf16x8 (&qop)[4], int qpos, int b) {
        f32x4 s0 = mfma_16x16x32_bf16(kop[0], qop[0], f32x4{0.f, 0.f, 0.f, 0.f});
        f32x4 s1 = mfma_16x16x32_bf16(kop[1], qop[1], f32x4{0.f, 0.f, 0.f, 0.f});
        s0 = mfma_16x16x32_bf16(kop[2], qop[2], s0);
        s1 = mfma_16x16x32_bf16(kop[3], qop[3], s1);
        f32x4 s = s0 + s1;
        // causal mask (it only bites in the query's own block; applied
        // without a branch so that two queries' products can interleave)
        const int key0 = b * kBlock + 16 * wave + 4 * l4;
#pragma unroll
        for (int r = 0; r < 4; ++r) s[r] = key0 + r > qpos ? -INFINITY : s[r];
        return s;
    };
    auto score = [&](const bf16x8 (&kop)[4], const char (*qs)[kQBytes], int p, int qpos, int b) {
        bf16x8 qop[4];
        load_q(qs, p, qop);
        return score_q(kop, qop, qpos, b);
    };
    // P = 2^(scale' s - ref) for this wave's keys -> bf16 into ps[p];
    // returns the largest exponent.
    auto write_p = [&](const f32x4& s, char (*ps)[kQBytes], int p, float ref) {
        float x[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = __builtin_fmaf(s[r], qk_scale, -ref);
        const uint32_t w01 = pack2_bf16(__builtin_amdgcn_exp2f(x[0]), __builtin_amdgcn_exp2f(x[1]));
        const uint32_t w23 = pack2_bf16(__builtin_amdgcn_exp2f(x[2]), __builtin_amdgcn_exp2f(x[3]));
        *reinterpret_cast<u32x2*>(ps[p] + pw_off) = u32x2{w01, w23};
        return fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    };
    // Probabilities above 2^kOverflow could leave the f32 / bf16 range in the
    // sums: such a step is recomputed against a raised reference.
    constexpr float kOverflow = 64.f;

    // Interval i, between barriers i - 1 and i: the scores and probabilities
    // of step i and the products O += P V of step i - 1, so that the two
    // overlap and each step costs one barrier.  ep, ec, en hold the entries
    // of steps i - 1, i, i + 1 and move on by one at the end.  Buffers by
    // parity: qs / ps / vs hold step i's queries, probabilities and V (copied
    // during this interval); po / vo step i - 1's probabilities and V; qo
    // receives step i + 1's queries once step i - 1 is finished with them.
    // kr holds step i's K and receives step i + 1's once the scores are done.
    auto interval = [&](int i, u32x4& ep, u32x4& ec, u32x4& en, char (*qs)[kQBytes], char (*qo)[kQBytes],
                        char (*ps)[kQBytes], char (*po)[kQBytes], char* vs, const char* vo, bf16x8 (&kr)[4]) {
        const bool has_s = i < n_steps;
        const bool has_pv = i >= 1;
        const bool more = i + 1 < n_steps;
        const int qpos0 = a.pos0 + static_cast<int>(q_first);

        // ---- step i - 1 overflowed (workgroup-uniform, rare): raise the
        // reference of its queries to max(ref, block max) and recompute its
        // probabilities (its queries are still in qo; its K is fetched
        // again); the accumulators are scaled by 2^(old - new) below.
        const bool redo = has_pv && redo_step[(i - 1) & 1] == i - 1;
        if (redo) {
            const int bp = static_cast<int>(ep[0]);
            const uint32_t mp = ep[1];
            const int npp = __builtin_popcount(mp);
            bf16x8 ko[4];
            load_k(ep, ko);
            uint32_t m = mp;
            for (int p = 0; p < npp; ++p) {
                const int t = __builtin_ctz(m);
                m &= m - 1u;
                const f32x4 s = score(ko, qo, p, qpos0 + t, bp);
                const float mx = max_xor32(max_xor16(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]))));
                if (lane < 16) pmax[p][l16][wave] = mx;
            }
            lds_barrier();
            m = mp;
            for (int p = 0; p < npp; ++p) {
                const int t = __builtin_ctz(m);
                m &= m - 1u;
                const f32x4 m0 = *reinterpret_cast<const f32x4*>(&pmax[p][l16][0]);
                const f32x4 m1 = *reinterpret_cast<const f32x4*>(&pmax[p][l16][4]);
                const float mb = fmaxf(fmaxf(fmaxf(m0[0], m0[1]), fmaxf(m0[2], m0[3])),
                                       fmaxf(fmaxf(m1[0], m1[1]), fmaxf(m1[2], m1[3]))) * qk_scale;
                const float old = m_ref[t][l16];
                const float ref = fmaxf(old, mb);
                write_p(score(ko, qo, p, qpos0 + t, bp), po, p, ref);
                if (wave == 0 && lane < 16) {
                    rnew[p][l16] = ref;
                    alph[p][l16] = __builtin_amdgcn_exp2f(old - ref);
                }
            }
            lds_barrier();                                      // every read of the old references is done
            if (wave == 0 && lane < 16) {
                m = mp;
                for (int p = 0; p < npp; ++p) {
                    const int t = __builtin_ctz(m);
                    m &= m - 1u;
                    m_ref[t][l16] = rnew[p][l16];
                }
            }
            lds_barrier();                                      // step i reads the new references
            __builtin_amdgcn_s_waitcnt(0);                      // (nothing of this path stays in flight)
        }
        // step i + 1's queries first (qo is free now): they have the whole
        // interval to land
        if (more) stage_queries(en, qo);

        // ---- step i: S, P for this wave's 16 keys, every query of the step
        if (has_s) {
            stage_v(ec, vs, 0);
            stage_v(ec, vs, 1);
        }
        float xmax = -INFINITY;
        if (has_s) {
            const int b = static_cast<int>(ec[0]);
            uint32_t m = ec[1];
            const int np = __builtin_popcount(m);
            // two queries per iteration, so that their read / product /
            // exponent chains overlap
            int p = 0;
            for (; p + 1 < np; p += 2) {
                const int t0 = __builtin_ctz(m);
                m &= m - 1u;
                const int t1 = __builtin_ctz(m);
                m &= m - 1u;
                const float r0 = m_ref[t0][l16], r1 = m_ref[t1][l16];
                bf16x8 q0[4], q1[4];
                load_q(qs, p, q0);
                load_q(qs, p + 1, q1);
                const f32x4 s0 = score_q(kr, q0, qpos0 + t0, b);
                const f32x4 s1 = score_q(kr, q1, qpos0 + t1, b);
                xmax = fmaxf(xmax, fmaxf(write_p(s0, ps, p, r0), write_p(s1, ps, p + 1, r1)));
            }
            if (p < np) {
                const int t = __builtin_ctz(m);
                xmax = fmaxf(xmax, write_p(score(kr, qs, p, qpos0 + t, b), ps, p, m_ref[t][l16]));
            }
        }
        if (more) load_k(en, kr);                               // step i's keys are no longer needed
        if (has_s) {
            stage_v(ec, vs, 2);
            stage_v(ec, vs, 3);
        }

        // ---- step i - 1: O^T += V^T P^T for this wave's 16 dims, every
        // query of the step, and the row sums of its own queries
        if (has_pv) {
            const uint32_t mask = ep[1];
            const int np = __builtin_popcount(mask);
            bf16x8 vop[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    LDS_PTR(v4i16, vo + kChunk * c * kRowBytes + voff));
                const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    LDS_PTR(v4i16, vo + (kChunk * c + 16) * kRowBytes + voff));
                vop[c] = __builtin_shufflevector(__builtin_bit_cast(bf16x4_t, lo), __builtin_bit_cast(bf16x4_t, hi),
                                                 0, 1, 2, 3, 4, 5, 6, 7);
            }
            // the next query's P operand is read as soon as this one's
            // products have been issued
            bf16x8 pt[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) pt[c] = *reinterpret_cast<const bf16x8*>(po[0] + pr_off + 1024 * c);
            int p = 0;
#pragma unroll
            for (int t = 0; t < kTq; ++t) {
                if ((mask >> t) & 1u) {                         // wave-uniform
                    const bool own = (t % kPaWaves) == wave;
                    if (redo) {
                        const float al = alph[p][l16];
                        acc[t] = acc[t] * al;
                        if (own) lsum[t / kPaWaves] *= al;
                    }
#pragma unroll
                    for (int c = 0; c < 4; ++c) acc[t] = mfma_16x16x32_bf16(vop[c], pt[c], acc[t]);
                    if (own) {
                        const bf16x2_t ones2 = __builtin_bit_cast(bf16x2_t, 0x3F803F80u);   // {1, 1}
                        float su = lsum[t / kPaWaves];
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            const u32x4 w = __builtin_bit_cast(u32x4, pt[c]);
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                const uint32_t wj = w[j];   // (a vector element is not an object to bit-cast)
                                su = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, wj), ones2, su, false);
                            }
                        }
                        lsum[t / kPaWaves] = su;
                    }
                    ++p;
                    if (p < np) {
#pragma unroll
                        for (int c = 0; c < 4; ++c) pt[c] = *reinterpret_cast<const bf16x8*>(po[p] + pr_off + 1024 * c);
                    }
                }
            }
        }
        if (__builtin_amdgcn_ballot_w64(xmax > kOverflow) != 0 && lane == 0) redo_step[i & 1] = i;
        // step i + 2's entry: a scalar load, issued last because every
        // wait for an LDS read would also wait for it
        u32x4 e2 = en;
        if (i + 2 < n_steps) e2 = steps_s[i + 2];
        // barrier i: step i's probabilities and V, step i + 1's K and
        // queries have landed
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        ep = ec;
        ec = en;
        en = e2;
    };

    bf16x8 kr[4];
    u32x4 ep = steps[0], ec = steps[0], en = steps[n_steps > 1 ? 1 : 0];   // every tile has a step (its local block)
    if (n_steps > 0) {
        load_k(ec, kr);
        stage_queries(ec, qbuf0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int i = 0; i <= n_steps; i += 2) {
        interval(i, ep, ec, en, qbuf0, qbuf1, pbuf0, pbuf1, vbuf0, vbuf1, kr);
        if (i + 1 > n_steps) break;
        interval(i + 1, ep, ec, en, qbuf1, qbuf0, pbuf1, pbuf0, vbuf1, vbuf0, kr);
    }
    // row sums to LDS: the owner wave adds its four lane groups' partial sums
#pragma unroll
    for (int k = 0; k < kTq / kPaWaves; ++k) {
        float su = lsum[k];
        su += __shfl_xor(su, 16, 64);
        su += __shfl_xor(su, 32, 64);
        if (lane < 16) l_fin[k * kPaWaves + wave][l16] = su;
    }
    __syncthreads();

    // ---- normalise and write: lane holds O^T[dim 16w + 4*l4 + r][head l16]
    float* dst = a.out + q_base + static_cast<int64_t>(l16) * kHeadDim + 16 * wave + 4 * l4;
#pragma unroll
    for (int t = 0; t < kTq; ++t) {
        if (t < n_tq) {
            const float inv = 1.f / l_fin[t][l16];
            *reinterpret_cast<f32x4*>(dst + t * kQStride) = acc[t] * inv;
        }
    }
}

int64_t n_tiles_of(int64_t n_q) { return (n_q + kTq - 1) / kTq; }

}  // namespace

size_t prefill_attend_ws_bytes(int64_t n_q, int top_k) {
    const int64_t n_wg = n_tiles_of(n_q) * kGroups;
    const size_t counts = (static_cast<size_t>(n_wg) * sizeof(int32_t) + 255) & ~size_t(255);
    return counts + static_cast<size_t>(n_wg) * kTq * top_k * sizeof(u32x4);
}

hipError_t launch_prefill_attend(const uint16_t* k, const uint16_t* v, const Pager& pg, const uint16_t* q,
                                 int32_t stream, int32_t pos0, int64_t n_q, const int32_t* sel, int top_k,
                                 float scale, float* out, void* ws, hipStream_t s) {
    const int64_t n_wg = n_tiles_of(n_q) * kGroups;
    const size_t counts_bytes = (static_cast<size_t>(n_wg) * sizeof(int32_t) + 255) & ~size_t(255);
    int32_t* counts = static_cast<int32_t*>(ws);
    u32x4* steps = reinterpret_cast<u32x4*>(static_cast<char*>(ws) + counts_bytes);
    const int nblk = (pos0 + static_cast<int>(n_q) - 1) / kBlock + 1;

    StepArgs sa;
    sa.sel = sel;
    sa.top_k = top_k;
    sa.pos0 = pos0;
    sa.n_q = n_q;
    sa.nblk = nblk;
    sa.max_steps = kTq * top_k;
    sa.pg = pg;
    sa.stream = stream;
    sa.counts = counts;
    sa.steps = steps;
    hipLaunchKernelGGL(prefill_steps_kernel, dim3(static_cast<unsigned>(n_wg)), dim3(kStepsThreads),
                       static_cast<size_t>(nblk) * sizeof(uint32_t), s, sa);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;

    PaArgs a;
    a.k = k;
    a.v = v;
    a.pg = pg;
    a.q = q;
    a.stream = stream;
    a.pos0 = pos0;
    a.n_q = n_q;
    a.last_row = pos0 + n_q - 1;
    a.max_steps = kTq * top_k;
    a.counts = counts;
    a.steps = steps;
    a.scale = scale;
    a.out = out;
    hipLaunchKernelGGL(prefill_attend_kernel, dim3(static_cast<unsigned>(n_wg)), dim3(kPaThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace msa
