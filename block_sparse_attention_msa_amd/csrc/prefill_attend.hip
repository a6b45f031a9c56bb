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
// local block, becomes several steps), and marks the blocks any tile uses;
// a second one copies K and V of each marked block into the order in which
// the matrix-core operands take them (64 KiB per block and group), so that
// the sweep loads every operand as whole contiguous KiB.
//
// Every step is spread evenly over all eight waves, whatever queries it
// holds: for S = Q K^T wave w takes keys 16w .. 16w+15 of the block for every
// query of the step and writes its bf16 probabilities to LDS; for O += P V
// wave w owns output dims 16w .. 16w+15 of all 32 queries of the tile, so the
// 16-head x 128-dim accumulators of the whole tile live in registers, one
// 16 x 16 slice per wave and query.  Both operands a wave needs from the
// block -- its 16 keys of K and its 16 dims of V^T, 4 KiB each -- are loaded
// from the rearranged copy straight into its registers: no K or V passes
// through LDS, and each wave waits only for its own loads.  K of the next
// step is loaded once this step's scores are formed, V^T of this step once
// the previous step's products are done, so each load has the other half of
// a step to land.  LDS carries only the step's queries (copied in with
// global_load_lds one step ahead) and the probabilities exchanged between
// the two halves.
//
// The softmax needs no exchange of maxima: each (query, head) uses one fixed
// reference for the whole sweep (its score against its own key, always
// selected), and a block whose probabilities would pass 2^64 is recomputed
// against a raised reference (rare).  The owner wave of each query sums the
// bf16 probabilities it reads as P V operands (v_dot2 against ones), so the
// normalisation sums exactly the weights applied.
//
// The sweep is pipelined by one step with a single barrier per step: the
// interval between barriers i - 1 and i holds the scores of step i and the
// products P V of step i - 1, with probabilities and the step's queries in
// two-deep LDS rings.
#include "common.hpp"

namespace msa {
namespace {

constexpr int kPaWaves = 8;
constexpr int kPaThreads = 64 * kPaWaves;
constexpr int kTq = 32;                     // queries per tile (one mask bit each)
constexpr int kPb = 8;                      // queries per step
constexpr int kRowBytes = kHeadDim * 2;     // one group's K or V row, one head's Q row: 256 B
constexpr int kVtElems = kBlock * kHeadDim;           // V^T of one block and group: 32 KiB
constexpr int kQBytes = kHeadsPerGroup * kRowBytes;  // 4 KiB: one query's 16 heads
constexpr float kLog2eP = 1.4426950408889634f;
constexpr int kStepsThreads = 256;
constexpr int kVtThreads = 256;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

// Query rows are stored with their 16 segments permuted by seg ^ f(row & 15),
// f a 4-bit rotate, one-to-one on 16 consecutive rows, so that the operand
// reads of 16 rows at one segment have no bank conflicts.
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
// table of a paged cache, so that the sweep does no table lookups.  Every
// block in the tile's union is marked in used[g][block] (cleared first by
// prefill_clear_kernel), so that only those blocks of V are transposed.
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
    uint32_t* used;
};

__global__ __launch_bounds__(256) void prefill_clear_kernel(uint32_t* used, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) used[i] = 0u;
}

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
        if (m == 0u) continue;
        a.used[g * a.nblk + b] = 1u;           // every tile that uses the block writes the same value
        const uint64_t row = static_cast<uint64_t>(a.pg.block_row(a.stream, b));
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
// K and V of the used blocks, rearranged into matrix-core operand order so
// that the sweep reads each wave's operands as four contiguous KiB (a load
// instruction then covers eight whole 128-byte lines; the 16 rows x 64 bytes
// of a load straight from the cache rows cost the load unit about 2.5 times
// as much).  Block b of group g occupies 2 * kVtElems bf16 at
// kv + (g * nblk + b) * 2 * kVtElems, each half 2048 slots of 16 bytes,
// slot (4w + c) * 64 + lane (lane = 16 * l4 + l16):
//   K half: K[key 16w + l16][dims 32c + 8*l4 .. +7], the A operand of wave
//           w's score product with dims 32c .. 32c + 31;
//   V half: V[key][dim 16w + l16] for keys 32c + 4*l4 + j (j = 0..3) and
//           32c + 16 + 4*l4 + j, the A operand of wave w's product with
//           chunk c of the probabilities, in the key order the score
//           products write them.
// Keys past the chunk's last key are zero (they are masked, and their
// probabilities are zero).  A quantized cache is dequantized here: each code
// times its 32-value block's f32 scale, formed in f32 and rounded once to
// bf16, so the sweep is the same for every cache format.
// ---------------------------------------------------------------------------
struct KvArgs {
    const void* k;          // bf16 rows, or codes (kv_format 1: int8, 2: 4-bit)
    const void* v;
    const float* k_scale;   // quantized caches: one f32 per 32 values of a group's row
    const float* v_scale;
    Pager pg;
    int32_t stream;
    int nblk;
    int last_row;
    const uint32_t* used;
    uint16_t* kv;
};

// The eight codes of dims 8 seg .. 8 seg + 7 of cache row `rg` (row x group)
// as exact floats: int8 bytes (kQ 1), or (kQ 2) the low nibbles (values
// 0 .. 15 of a 32-value block) or high nibbles (values 16 .. 31), stored + 8,
// of eight bytes.
template <int kQ>
__device__ __forceinline__ void row_codes8(const void* base, int64_t rg, int seg, float* f) {
    const uint8_t* b = static_cast<const uint8_t*>(base);
    if constexpr (kQ == 1) {
        const u32x2 w = *reinterpret_cast<const u32x2*>(b + rg * kHeadDim + 8 * seg);
#pragma unroll
        for (int j = 0; j < 8; ++j) f[j] = static_cast<float>(static_cast<int8_t>((w[j >> 2] >> (8 * (j & 3))) & 255u));
    } else {
        const int j0 = 8 * (seg & 3);                   // first value inside the 32-value block
        const u32x2 w = *reinterpret_cast<const u32x2*>(b + rg * (kHeadDim / 2) + 16 * (seg >> 2) + (j0 & 15));
        const int sh = (j0 & 16) ? 4 : 0;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            f[j] = static_cast<float>(static_cast<int>((w[j >> 2] >> (8 * (j & 3) + sh)) & 15u) - 8);
    }
}

// Dims 8 seg .. 8 seg + 7 of cache row `rg` as eight bf16 values.
template <int kQ>
__device__ __forceinline__ u32x4 row_segment(const void* base, const float* scale, int64_t rg, int seg) {
    if constexpr (kQ == 0) {
        return *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + rg * kHeadDim + 8 * seg);
    } else {
        float f[8];
        row_codes8<kQ>(base, rg, seg, f);
        const float sc = scale[rg * (kHeadDim / 32) + (seg >> 2)];
        return u32x4{pack2_bf16(f[0] * sc, f[1] * sc), pack2_bf16(f[2] * sc, f[3] * sc),
                     pack2_bf16(f[4] * sc, f[5] * sc), pack2_bf16(f[6] * sc, f[7] * sc)};
    }
}

// Workgroup (g, b, m) handles keys 32m .. 32m + 31 of block b: the K slots of
// waves w = 2m, 2m + 1 and the V slots of chunk c = m, 8 KiB each way.
template <int kQ>
__global__ __launch_bounds__(kVtThreads) void prefill_kv_kernel(KvArgs a) {
    const int m = blockIdx.x & 3;
    const int g = (blockIdx.x >> 2) % kGroups;
    const int b = (blockIdx.x >> 2) / kGroups;
    if (a.used[g * a.nblk + b] == 0u) return;           // workgroup-uniform
    constexpr int kPitch = kHeadDim + 8;                 // 272-byte rows: the gathers below hit distinct banks
    __shared__ __attribute__((aligned(16))) uint16_t tv[32][kPitch];
    const int64_t row0 = a.pg.block_row(a.stream, b) + 32 * m;
    const int key0 = b * kBlock + 32 * m;
    uint16_t* dst = a.kv + (static_cast<int64_t>(g) * a.nblk + b) * 2 * kVtElems;
    // 32 rows x 16 segments of K and of V: thread t takes segments t and t + 256
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int s = threadIdx.x + kVtThreads * h;
        const int r = s >> 4, seg = s & 15;
        u32x4 xk = u32x4{0u, 0u, 0u, 0u}, xv = xk;
        if (key0 + r <= a.last_row) {
            const int64_t rg = (row0 + r) * kGroups + g;
            xk = row_segment<kQ>(a.k, a.k_scale, rg, seg);
            xv = row_segment<kQ>(a.v, a.v_scale, rg, seg);
        }
        // K: key 32m + r = 16w + l16 with w = 2m + r / 16, dims 8 seg = 32c + 8 l4
        const int w = 2 * m + (r >> 4), l16 = r & 15, c = seg >> 2, l4 = seg & 3;
        *reinterpret_cast<u32x4*>(dst + 8 * ((4 * w + c) * 64 + 16 * l4 + l16)) = xk;
        *reinterpret_cast<u32x4*>(&tv[r][8 * seg]) = xv;
    }
    __syncthreads();
    // V^T slots of chunk m: (4w + m) * 64 + lane for the eight waves w
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int o = threadIdx.x + kVtThreads * h;     // 0 .. 511
        const int lane = o & 63, w = o >> 6;
        const int l16 = lane & 15, l4 = lane >> 4;
        const int dim = 16 * w + l16;
        const int k0 = 4 * l4;
        uint32_t x[4];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            x[j] = static_cast<uint32_t>(tv[k0 + 2 * j][dim]) | (static_cast<uint32_t>(tv[k0 + 2 * j + 1][dim]) << 16);
            x[2 + j] = static_cast<uint32_t>(tv[k0 + 16 + 2 * j][dim]) |
                       (static_cast<uint32_t>(tv[k0 + 16 + 2 * j + 1][dim]) << 16);
        }
        *reinterpret_cast<u32x4*>(dst + kVtElems + 8 * ((4 * w + m) * 64 + lane)) = u32x4{x[0], x[1], x[2], x[3]};
    }
}

// ---------------------------------------------------------------------------
// Attention sweep.
// ---------------------------------------------------------------------------
struct PaArgs {
    const void* k;          // the cache's K rows (bf16, or codes), for the softmax references
    const float* k_scale;   // quantized caches: one f32 per 32 values
    int kv_format;          // 0 bf16, 1 int8, 2 4-bit
    const uint16_t* kv;
    Pager pg;
    const uint16_t* q;
    int32_t stream;
    int32_t pos0;
    int64_t n_q;
    int nblk;
    int max_steps;
    const int32_t* counts;
    const u32x4* steps;
    float scale;
    float* out;
};

// Waits until at most 4 vector-memory loads of this wave are in flight (the
// four V^T loads issued last), its LDS accesses are done, then the
// workgroup barrier.  Loads return in issue order, so everything issued
// before those four -- the next step's query copies and keys -- has landed.
__device__ __forceinline__ void step_barrier() {
    __builtin_amdgcn_s_waitcnt(0x0074);        // vmcnt 4, expcnt 7, lgkmcnt 0
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

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

    // Two-deep rings (by step parity) for the step's queries and its
    // probabilities.  Separate objects, so that reads of one are not made to
    // wait for copies in flight into another.
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
            const int64_t rg = a.pg.row(a.stream, a.pos0 + static_cast<int>(q_first) + t) * kGroups + g;
            float s0 = 0.f, s1 = 0.f;
            if (a.kv_format == 0) {
                const uint16_t* kr = static_cast<const uint16_t*>(a.k) + rg * kHeadDim;
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
            } else {
                // codes times their block's scale (any finite reference will do)
#pragma unroll 1
                for (int seg = 0; seg < kHeadDim / 8; ++seg) {
                    float f[8];
                    if (a.kv_format == 1) row_codes8<1>(a.k, rg, seg, f);
                    else row_codes8<2>(a.k, rg, seg, f);
                    const u32x4 qa = *reinterpret_cast<const u32x4*>(qr + 8 * seg);
                    float p = 0.f;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        p = __builtin_fmaf(__uint_as_float(qa[j] << 16), f[2 * j], p);
                        p = __builtin_fmaf(__uint_as_float(qa[j] & 0xffff0000u), f[2 * j + 1], p);
                    }
                    s0 = __builtin_fmaf(p, a.k_scale[rg * (kHeadDim / 32) + (seg >> 2)], s0);
                }
            }
            r = (s0 + s1) * qk_scale;
        }
        m_ref[t][h] = r;
        if (threadIdx.x < 2) redo_step[threadIdx.x] = -1;
    }
    // O^T slices (dims 16w + 4*l4 + r, head l16) of all tile queries, and
    // the row sums of the queries t with t % 8 == w: lane (l16, l4) sums the
    // bf16 probabilities of head l16 it reads as operands, so that the
    // normalisation sums exactly the weights applied
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
    // P exchange: chunk c = keys 32c .. 32c+31 is written by waves 2c (keys
    // 32c + 4*l4 + r) and 2c+1 (keys 32c + 16 + 4*l4 + r) and read as the
    // 8-key B operand of lane (l16, l4) of every wave; V^T holds the same
    // key order.
    const int pw_off = (((wave >> 1) * 4 + l4) * 16 + l16) * 16 + (wave & 1) * 8;
    const int pr_off = (l4 * 16 + l16) * 16;   // + 1 KiB per chunk

    // e: a step entry (block id, mask, first cache row).  This wave's
    // operands of the block from the rearranged copy, four contiguous KiB
    // each: K of keys 16w .. 16w + 15 (kr[c] the A operand of the score
    // product over dims 32c .. 32c + 31) and V^T of dims 16w .. 16w + 15
    // (vr[c] the A operand of the product with probability chunk c).
    const uint16_t* kv_g = a.kv + static_cast<int64_t>(g) * a.nblk * 2 * kVtElems + (wave * 4 * 64 + lane) * 8;
    auto load_k = [&](const u32x4& e, bf16x8 (&kr)[4]) {
        const uint16_t* src = kv_g + static_cast<int64_t>(e[0]) * 2 * kVtElems;
#pragma unroll
        for (int c = 0; c < 4; ++c) kr[c] = *reinterpret_cast<const bf16x8*>(src + c * 64 * 8);
    };
    auto load_v = [&](const u32x4& e, bf16x8 (&vr)[4]) {
        const uint16_t* src = kv_g + static_cast<int64_t>(e[0]) * 2 * kVtElems + kVtElems;
#pragma unroll
        for (int c = 0; c < 4; ++c) vr[c] = *reinterpret_cast<const bf16x8*>(src + c * 64 * 8);
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
    // parity: qs / ps hold step i's queries and probabilities; po step
    // i - 1's probabilities; qo receives step i + 1's queries once step
    // i - 1 is finished with them.  kr holds step i's K and receives step
    // i + 1's once the scores are done; vr holds step i - 1's V^T and
    // receives step i's once the products are done.
    auto interval = [&](int i, u32x4& ep, u32x4& ec, u32x4& en, char (*qs)[kQBytes], char (*qo)[kQBytes],
                        char (*ps)[kQBytes], char (*po)[kQBytes], bf16x8 (&kr)[4], bf16x8 (&vr)[4]) {
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
        // step i + 1's keys (or, past the end, step i's again: the loads are
        // unconditional so that the wait counts stay static)
        load_k(en, kr);

        // ---- step i - 1: O^T += V^T P^T for this wave's 16 dims, every
        // query of the step, and the row sums of its own queries
        if (has_pv) {
            // this wave's V^T of step i - 1 (loaded before this interval's
            // query copies and keys) is in place once at most the four key
            // loads are outstanding
            __builtin_amdgcn_s_waitcnt(0x0074);         // vmcnt 4, expcnt 7, lgkmcnt 0
            const uint32_t mask = ep[1];
            const int np = __builtin_popcount(mask);
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
                    for (int c = 0; c < 4; ++c) acc[t] = mfma_16x16x32_bf16(vr[c], pt[c], acc[t]);
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
        // step i's V^T for the products of the next interval (past the end:
        // the last step's again)
        load_v(ec, vr);
        if (__builtin_amdgcn_ballot_w64(xmax > kOverflow) != 0 && lane == 0) redo_step[i & 1] = i;
        // step i + 2's entry: a scalar load, issued last because every
        // wait for an LDS read would also wait for it
        u32x4 e2 = en;
        if (i + 2 < n_steps) e2 = steps_s[i + 2];
        // barrier i: step i's probabilities, step i + 1's queries and keys
        // are in place (step i's V^T may still be on its way)
        step_barrier();
        ep = ec;
        ec = en;
        en = e2;
    };

    // (every tile has a step, its local block, when the selection holds it;
    // a tile without steps skips the sweep rather than read an entry)
    if (n_steps > 0) {
        bf16x8 kr[4], vr[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) vr[c] = bf16x8{};   // first loaded at the end of interval 0
        u32x4 ep = steps[0], ec = steps[0], en = steps[n_steps > 1 ? 1 : 0];
        load_k(ec, kr);
        stage_queries(ec, qbuf0);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        for (int i = 0; i <= n_steps; i += 2) {
            interval(i, ep, ec, en, qbuf0, qbuf1, pbuf0, pbuf1, kr, vr);
            if (i + 1 > n_steps) break;
            interval(i + 1, ep, ec, en, qbuf1, qbuf0, pbuf1, pbuf0, kr, vr);
        }
        __builtin_amdgcn_s_waitcnt(0);                  // the last (unused) loads
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
size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

// Workspace layout: step counts [n_wg] i32 | used flags [4][nblk] u32 |
// step lists [n_wg][kTq * top_k] of 16 bytes | rearranged K and V
// [4][nblk][2][kVtElems] bf16.
struct WsLayout {
    size_t counts, used, steps, kv, total;
};
WsLayout ws_layout(int64_t n_q, int top_k, int nblk) {
    const int64_t n_wg = n_tiles_of(n_q) * kGroups;
    WsLayout l;
    l.counts = 0;
    l.used = align256(static_cast<size_t>(n_wg) * sizeof(int32_t));
    l.steps = l.used + align256(static_cast<size_t>(kGroups) * nblk * sizeof(uint32_t));
    l.kv = l.steps + align256(static_cast<size_t>(n_wg) * kTq * top_k * sizeof(u32x4));
    l.total = l.kv + static_cast<size_t>(kGroups) * nblk * 2 * kVtElems * sizeof(uint16_t);
    return l;
}

}  // namespace

size_t prefill_attend_ws_bytes(int64_t n_q, int top_k, int32_t max_pos) {
    return ws_layout(n_q, top_k, max_pos / kBlock + 1).total;
}

hipError_t launch_prefill_attend(const void* k, const void* v, int kv_format, const float* k_scale,
                                 const float* v_scale, const Pager& pg, const uint16_t* q, int32_t stream,
                                 int32_t pos0, int64_t n_q, const int32_t* sel, int top_k, float scale, float* out,
                                 void* ws, hipStream_t s) {
    const int64_t n_wg = n_tiles_of(n_q) * kGroups;
    const int last_row = static_cast<int>(pos0 + n_q - 1);
    const int nblk = last_row / kBlock + 1;
    const WsLayout l = ws_layout(n_q, top_k, nblk);
    char* base = static_cast<char*>(ws);
    int32_t* counts = reinterpret_cast<int32_t*>(base + l.counts);
    uint32_t* used = reinterpret_cast<uint32_t*>(base + l.used);
    u32x4* steps = reinterpret_cast<u32x4*>(base + l.steps);
    uint16_t* kv = reinterpret_cast<uint16_t*>(base + l.kv);

    const int n_used = kGroups * nblk;
    hipLaunchKernelGGL(prefill_clear_kernel, dim3(static_cast<unsigned>((n_used + 255) / 256)), dim3(256), 0, s,
                       used, n_used);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;

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
    sa.used = used;
    hipLaunchKernelGGL(prefill_steps_kernel, dim3(static_cast<unsigned>(n_wg)), dim3(kStepsThreads),
                       static_cast<size_t>(nblk) * sizeof(uint32_t), s, sa);
    err = hipGetLastError();
    if (err != hipSuccess) return err;

    KvArgs ka;
    ka.k = k;
    ka.v = v;
    ka.k_scale = k_scale;
    ka.v_scale = v_scale;
    ka.pg = pg;
    ka.stream = stream;
    ka.nblk = nblk;
    ka.last_row = last_row;
    ka.used = used;
    ka.kv = kv;
    const dim3 kv_grid(static_cast<unsigned>(4 * n_used));
    switch (kv_format) {
        case 0: hipLaunchKernelGGL(prefill_kv_kernel<0>, kv_grid, dim3(kVtThreads), 0, s, ka); break;
        case 1: hipLaunchKernelGGL(prefill_kv_kernel<1>, kv_grid, dim3(kVtThreads), 0, s, ka); break;
        case 2: hipLaunchKernelGGL(prefill_kv_kernel<2>, kv_grid, dim3(kVtThreads), 0, s, ka); break;
        default: return hipErrorInvalidValue;
    }
    err = hipGetLastError();
    if (err != hipSuccess) return err;

    PaArgs a;
    a.k = k;
    a.k_scale = k_scale;
    a.kv_format = kv_format;
    a.kv = kv;
    a.pg = pg;
    a.q = q;
    a.stream = stream;
    a.pos0 = pos0;
    a.n_q = n_q;
    a.nblk = nblk;
    a.max_steps = kTq * top_k;
    a.counts = counts;
    a.steps = steps;
    a.scale = scale;
    a.out = out;
    hipLaunchKernelGGL(prefill_attend_kernel, dim3(static_cast<unsigned>(n_wg)), dim3(kPaThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace msa
