// attend.hip -- softmax attention over the selected keys only.
//
// "Add MiniMax-M3 (MSA: MiniMax Sparse Attention) support", Overview and
// Implementation: after selection, each query head attends over the keys of
// its group's selected blocks (16 x 128 = 2048 keys) instead of the context;
// "deepseek2 : GLM-DSA sparse attention (lightning indexer)", What this does:
// the same over the kept token ids.
//
// Design (gfx950):
//  * One workgroup of four wavefronts per (query, group, split), sized so the
//    grid is about one workgroup per compute unit.  A split owns a run of
//    128-key units: selected blocks (MSA) or 128 kept token ids (DSA).  The 16
//    query heads of a group are the N = 16 side of v_mfma_f32_16x16x32_bf16,
//    so a group's heads share every K/V byte that is read.
//  * Units stream HBM -> LDS with global_load_lds (no registers) into a ring
//    of two: the next unit's 64 KiB are in flight while the current one is
//    computed, nothing is gathered into a separate buffer.  Rows are stored
//    with their 16-byte segments permuted by the row index, so K operand reads
//    and the transposing V reads (ds_read_b64_tr_b16, which hand each lane
//    four consecutive keys of one dim) are free of bank conflicts.
//  * Wave w takes keys 32w .. 32w+31 of every unit: S^T = K Q^T (keys x
//    heads) leaves P^T in the layout O^T = V^T P^T wants.  Online softmax in
//    the log2 domain per wave; the four waves merge in LDS; splits write
//    (m, l, acc) partials that a second kernel combines in a fixed order, so
//    results are deterministic.
//  * Quantized caches (int8 or 4-bit codes, one f32 scale per 32 values; the
//    Strata compare page's int8 / Q4_0 KV): a unit's codes and scales are
//    loaded into registers while the previous unit is computed, then written
//    to the ring buffer in the same permuted layout as their codes (exact in
//    bf16) with the scales beside them: K's scales multiply each 32-dim
//    slice of S^T = K Q^T after its matrix-core product (one slice is one
//    scale block), and V's are folded into the probabilities, one bf16 P
//    operand per 32-dim block of the output, so the only rounding is that of
//    the scaled probabilities, as in the bf16 path.  4-bit codes enter
//    biased, as c + 136 (bf16 bits 0x4300 | nibble, two bit operations per
//    pair instead of a conversion per value): each score slice subtracts
//    136 x the sum of its query values before its scale, and the output
//    subtracts 136 x the sum of the bf16 probabilities it applied (kept per
//    lane and rescaled with the accumulators, subtracted once at the end).
#include "common.hpp"
#include "topk_regs.hpp"

namespace msa {
namespace {

constexpr int kAttWaves = 4;
constexpr int kAttThreads = 64 * kAttWaves;
constexpr int kUnit = 128;                        // keys per streamed unit
constexpr int kRowBytes = kHeadDim * 2;           // one group's K or V row: 256 B
constexpr int kUnitBytes = kUnit * kRowBytes;     // 32 KiB of K (and of V) per unit
constexpr int kCopiesPerUnit = kUnitBytes / 16 / kAttThreads;   // 16-byte copies per thread, K or V
constexpr int kPartFloats = kHeadsPerGroup * kHeadDim + 2 * kHeadsPerGroup;   // acc + (m, l)
constexpr float kLog2e = 1.4426950408889634f;
// Largest id list one split stages: a split streams at most 8 units (see
// attend_num_splits), i.e. 1024 DSA tokens or 8 MSA blocks.
constexpr int kMaxSplitEntries = 8 * kUnit;

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

// Segment permutation of a staged row (see the design note).
__device__ __forceinline__ int rowperm(int row) { return ((row & 7) << 1) | ((row >> 3) & 1); }
__device__ __forceinline__ int swz(int row, int seg) { return row * kRowBytes + ((seg ^ rowperm(row)) << 4); }

// Barrier ordering LDS accesses only: copies into LDS still in flight
// (counted by vmcnt) are not waited for.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);        // vmcnt 63, expcnt 7, lgkmcnt 0
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (expcnt and lgkmcnt left at their maxima).
constexpr unsigned waitcnt_vm(int n) {
    return static_cast<unsigned>((n & 15) | (((n >> 4) & 3) << 14) | (7 << 4) | (15 << 8));
}
static_assert(waitcnt_vm(0) == 0x0F70 && waitcnt_vm(16) == 0x4F70, "gfx9 s_waitcnt layout");

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), bf16x2_t));
}

struct KernelArgs {
    AttendArgs a;
    int n_split;
    int n_units;           // units per (query, group)
    int units_per_split;
};

// kMaxUnits: the units a split streams.  The unit loop is fully unrolled and
// every copy and wait in it is unconditional (units past the split's valid
// ones are copied from a valid row and fully masked), so the compiler can
// tell which ring buffer every copy in flight targets and reads of the other
// buffer never wait for it.
template <bool kTokenIds, int kMaxUnits, int kQ = 0>
__global__ __launch_bounds__(kAttThreads, 1) void attend_kernel(KernelArgs ka) {
    const AttendArgs& a = ka.a;
    const int64_t wg = blockIdx.x;                 // ((query * kGroups) + group) * n_split + split
    const int sp = static_cast<int>(wg % ka.n_split);
    const int g = static_cast<int>((wg / ka.n_split) % kGroups);
    const int64_t i = wg / (static_cast<int64_t>(ka.n_split) * kGroups);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int l16 = lane & 15;
    const int l4 = lane >> 4;

    // ring of two units; separate objects, so that reads of one are not made
    // to wait for the copies in flight into the other
    __shared__ __attribute__((aligned(16))) char kbuf0[kUnitBytes];
    __shared__ __attribute__((aligned(16))) char kbuf1[kUnitBytes];
    __shared__ __attribute__((aligned(16))) char vbuf0[kUnitBytes];
    __shared__ __attribute__((aligned(16))) char vbuf1[kUnitBytes];
    __shared__ int32_t sel_s[kMaxSplitEntries];    // this split's ids
    __shared__ int32_t row_s[kMaxSplitEntries + 1];   // their cache rows (MSA: a block's first row), then the query's own
    __shared__ float mrg_m[kAttWaves][kHeadsPerGroup];
    __shared__ float mrg_l[kAttWaves][kHeadsPerGroup];
    __shared__ int n_valid_s;
    // quantized K and V: scales of the ring's two units, [block][key] (4 keys of a lane contiguous)
    __shared__ __attribute__((aligned(16))) float kscl_s[2][kQ ? 4 * kUnit : 4];
    __shared__ __attribute__((aligned(16))) float vscl_s[2][kQ ? 4 * kUnit : 4];

    const int64_t s = a.stream ? a.stream[i] : a.stream0;
    const int p = a.stream ? a.pos[i] : a.pos0 + static_cast<int>(i);
    const int32_t* sel = a.sel + i * static_cast<int64_t>(a.sel_len) * (kTokenIds ? 1 : kGroups) +
                         g * a.sel_g_stride;
    const uint16_t* kg = a.k + g * kHeadDim;   // cache row r at + r*kGroups*kHeadDim
    const uint16_t* vg = a.v + g * kHeadDim;
    const Pager pg = a.pg;
    const int own_row = static_cast<int>(pg.row(s, p));   // cache rows fit int32 (< 2 TiB of K)
    constexpr int kRow = kGroups * kHeadDim;

    // this split's units and their ids (ascending, -1 padding at the end)
    const int u_begin = sp * ka.units_per_split;
    const int u_end = min(u_begin + ka.units_per_split, ka.n_units);
    const int e_begin = kTokenIds ? u_begin * kUnit : u_begin;
    const int e_end = kTokenIds ? min(u_end * kUnit, a.sel_len) : u_end;
    // Q^T operand: B[k = dim][n = head]; lane: head l16, dims 32*ks + 8*l4 + 0..7
    // (loaded with the ids, before any copy into LDS is in flight)
    bf16x8 qb[4];
    {
        const uint16_t* qrow = a.q + (i * kGroups * kHeadsPerGroup + g * kHeadsPerGroup + l16) * kHeadDim;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qb[ks] = *reinterpret_cast<const bf16x8*>(qrow + 32 * ks + 8 * l4);
    }
    if (threadIdx.x == 0) {
        n_valid_s = 0;
        row_s[kMaxSplitEntries] = own_row;
    }
    // decode step: this (query, group)'s blocks ranked here from the scan's
    // block scores (or a fine scan's partial maxima) by one wave, with the
    // keys of the block top-k (local block first, then the score, then the
    // lower id): up to 64 candidates by rank (the number of larger keys),
    // more by the top-k's register rounds; the winners in ascending id order
    constexpr int kRankDirect = 64;
    __shared__ uint64_t rkey_s[kRankDirect];
    __shared__ int32_t ranked_s[kMaxTopkBlocks];
    __shared__ int32_t chosen_s[kMaxTopkBlocks];
    const bool ranked = !kTokenIds && kQ == 0 && a.bs_part != nullptr;     // launch-uniform
    if constexpr (!kTokenIds && kQ == 0) {
        if (ranked) {
            const int loc = p / kBlock;
            const int nvis = loc + 1;                   // <= nblk_part <= kRankedBlocks
            const int k = min(a.sel_len, nvis);
            const float* row = a.bs_part + (i * kGroups + g) * a.nblk_part * a.n_sub;
            if (nvis <= kRankDirect) {
                uint64_t key = 0;
                if (wave == 0) {
                    if (lane < nvis) {
                        const float* bp = row + lane * a.n_sub;
                        float sc = bp[0];
                        for (int e = 1; e < a.n_sub; ++e) sc = fmaxf(sc, bp[e]);
                        key = (static_cast<uint64_t>(ordered_key(sc)) << 31) |
                              static_cast<uint64_t>(0x7fffffff - lane) | (lane == loc ? 1ull << 63 : 0ull);
                    }
                    rkey_s[lane] = key;
                }
                __syncthreads();
                if (wave == 0) {
                    int rank = 0;
                    for (int c = 0; c < nvis; ++c) rank += rkey_s[c] > key;
                    const bool win = lane < nvis && rank < k;
                    const uint64_t wins = __builtin_amdgcn_ballot_w64(win);
                    if (win) ranked_s[__builtin_popcountll(wins & ((1ull << lane) - 1ull))] = lane;
                    for (int t = k + lane; t < a.sel_len; t += 64) ranked_s[t] = -1;
                }
            } else {
                if (wave == 0) {
                    auto rank_regs = [&](auto per) __attribute__((always_inline)) {
                        constexpr int kPer = decltype(per)::value;
                        float pre[kPer];
#pragma unroll
                        for (int j = 0; j < kPer; ++j) {
                            const int b = lane + 64 * j;
                            pre[j] = row[(b < a.nblk_part ? b : 0) * a.n_sub];
                        }
                        topk_in_registers<kPer, (kPer > 8)>(row, pre, a.n_sub, nvis, loc, k, lane, chosen_s);
                    };
                    if (nvis <= 256) rank_regs(std::integral_constant<int, 4>{});
                    else if (nvis <= 512) rank_regs(std::integral_constant<int, 8>{});
                    else rank_regs(std::integral_constant<int, 16>{});   // one score per block (coarse scan)
                }
                __syncthreads();
                if (wave == 0) write_ascending(chosen_s, k, a.sel_len, lane, ranked_s);
            }
            __syncthreads();
            if (sp == 0) {
                for (int t = threadIdx.x; t < a.sel_len; t += kAttThreads)
                    a.sel_out[(i * kGroups + g) * a.sel_len + t] = ranked_s[t];
                if (threadIdx.x == 0) a.n_sel_out[i * kGroups + g] = k;
            }
        }
    }
    __syncthreads();
    for (int e = e_begin + static_cast<int>(threadIdx.x); e < e_begin + (u_end - u_begin) * (kTokenIds ? kUnit : 1);
         e += kAttThreads) {
        int id = e < e_end ? (ranked ? ranked_s[e] : sel[e]) : -1;
        if (kTokenIds ? (id > p) : (id > p / kBlock)) id = -1;
        sel_s[e - e_begin] = id;
        row_s[e - e_begin] = id < 0 ? own_row
                                    : static_cast<int>(kTokenIds ? pg.row(s, id) : pg.block_row(s, id));
        // units are valid up to the first unit whose first id is padding
        if (id >= 0 && (kTokenIds ? ((e - e_begin) % kUnit == 0) : true))
            atomicMax(&n_valid_s, (e - e_begin) / (kTokenIds ? kUnit : 1) + 1);
    }
    __syncthreads();
    const int n_units = n_valid_s;                  // the split size guarantees n_valid_s <= kMaxUnits
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));      // the query operand has arrived
    const float qk_scale = a.scale * kLog2e;

    // Copies of unit u into (kd, vd): slot c = 256*j + thread holds segment
    // (c % 16) ^ f(row) of row c / 16; rows whose key is padding or past the
    // query read the query's own row (finite, masked below).
    auto stage = [&](int u, char* kd, char* vd) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < kCopiesPerUnit; ++j) {
            const int c = kAttThreads * j + static_cast<int>(threadIdx.x);
            const int row = c >> 4;
            const int seg = (c & 15) ^ rowperm(row);
            // every read is an unconditional LDS read (in bounds for every
            // u < kMaxUnits; the query's own row sits past the entries), so
            // that no select between LDS and other memory becomes a flat load
            const int e = kTokenIds ? u * kUnit + row : u;
            const int tok = kTokenIds ? sel_s[e] : sel_s[e] * kBlock + row;
            const int r_e = row_s[e];
            const int r_own = row_s[kMaxSplitEntries];
            const bool bad = u >= n_units || tok < 0 || tok > p;
            const int crow = bad ? r_own : r_e + (kTokenIds ? 0 : row);
            const int64_t off = static_cast<int64_t>(crow) * kRow + 8 * seg;
            __builtin_amdgcn_global_load_lds(kg + off, LDS_PTR(void, kd + (kAttThreads * j + 64 * wave) * 16), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(vg + off, LDS_PTR(void, vd + (kAttThreads * j + 64 * wave) * 16), 16, 0, 0);
        }
    };

    // Quantized caches: a unit's codes are loaded in 16-byte chunks, eight
    // (int8: 128-byte rows) or four (4-bit: 64-byte rows) lanes per row, so
    // that one load instruction covers whole 128-byte lines, plus one 16-byte
    // load of a row's four block scales for K and for V by the threads
    // tid < kUnit.  Chunk c = kAttThreads * j + tid of K (and of V) is
    // (row c / 8, values 16 * (c % 8) ..) for int8, (row c / 4, scale block
    // c % 4) for 4-bit.
    constexpr int kQPerRow = kQ == 2 ? 4 : 8;                 // chunks per row
    constexpr int kQChunks = kQ ? kUnit * kQPerRow / kAttThreads : 1;
    // two register sets: unit u + 1 loads at the release of unit u - 1 and
    // is written to the ring after the math of unit u
    u32x4 kc[2][kQChunks], vc[2][kQChunks];
    f32x4 kscl[2], vscl[2];
    // cache row of key `row` of unit u (padding and keys past the query read
    // the query's own row: finite, and masked)
    auto qrow = [&](int u, int row) __attribute__((always_inline)) {
        const int e = kTokenIds ? u * kUnit + row : u;
        const int tok = kTokenIds ? sel_s[e] : sel_s[e] * kBlock + row;
        const int r_e = row_s[e];
        const int r_own = row_s[kMaxSplitEntries];
        const bool bad = u >= n_units || tok < 0 || tok > p;
        return static_cast<int64_t>(bad ? r_own : r_e + (kTokenIds ? 0 : row)) * kGroups + g;
    };
    auto qload = [&](int u, int set) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < kQChunks; ++j) {
            const int c = kAttThreads * j + static_cast<int>(threadIdx.x);
            const int64_t boff = qrow(u, c / kQPerRow) * (kQ == 1 ? kHeadDim : kHeadDim / 2) + 16 * (c % kQPerRow);
            kc[set][j] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(a.k) + boff);
            vc[set][j] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(a.v) + boff);
        }
        if (threadIdx.x < kUnit) {                 // waves 0, 1: one row's scales each
            const int64_t rq = qrow(u, static_cast<int>(threadIdx.x));
            kscl[set] = *reinterpret_cast<const f32x4*>(a.k_scale + rq * (kHeadDim / 32));
            vscl[set] = *reinterpret_cast<const f32x4*>(a.v_scale + rq * (kHeadDim / 32));
        }
    };
    // 8 codes -> 8 bf16 values (exact): int8 bytes, or the low / high
    // nibbles n (the code plus 8) of 8 bytes.  A nibble enters biased, as
    // 128 + n (bf16 bits 0x4300 | n, so a pair is one byte permute and one
    // and-or); the scores and the output subtract the bias's share after
    // their products (kQBias below).
    auto codes8 = [&](uint32_t w0, uint32_t w1, int mode) __attribute__((always_inline)) {
        if (mode != 0) {
            u32x4 r;
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const uint32_t w = h < 2 ? w0 : w1;
                // bytes 2 (h % 2), 2 (h % 2) + 1 of w at bits 0..7 and 16..23
                uint32_t pr = __builtin_amdgcn_perm(0u, w, (h & 1) ? 0x0c030c02u : 0x0c010c00u);
                if (mode == 2) pr >>= 4;
                // (pr & 0x000f000f) | 0x43004300 in one instruction (VOP3 takes no
                // literal here, so both constants sit in registers)
                uint32_t o;
                asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(o) : "v"(pr), "v"(0x000f000fu), "v"(0x43004300u));
                r[h] = o;
            }
            return r;
        }
        float f[8];
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const uint32_t word = b < 4 ? w0 : w1;
            const int byte = static_cast<int>((word >> (8 * (b & 3))) & 0xffu);
            f[b] = static_cast<float>(static_cast<int8_t>(byte));
        }
        return u32x4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                     pack_bf16x2(f[6], f[7])};
    };
    // 16 bytes of codes -> their 8-value segments of the staged row (the
    // ring's permuted layout)
    auto put_codes = [&](char* d, const u32x4& w, int c) __attribute__((always_inline)) {
        const int row = c / kQPerRow, part = c % kQPerRow;
        if constexpr (kQ == 1) {                   // values 16 part .. + 15: segments 2 part, 2 part + 1
            *reinterpret_cast<u32x4*>(d + swz(row, 2 * part)) = codes8(w[0], w[1], 0);
            *reinterpret_cast<u32x4*>(d + swz(row, 2 * part + 1)) = codes8(w[2], w[3], 0);
        } else {                                   // block `part`: values 0..15 low nibbles, 16..31 high
            *reinterpret_cast<u32x4*>(d + swz(row, 4 * part)) = codes8(w[0], w[1], 1);
            *reinterpret_cast<u32x4*>(d + swz(row, 4 * part + 1)) = codes8(w[2], w[3], 1);
            *reinterpret_cast<u32x4*>(d + swz(row, 4 * part + 2)) = codes8(w[0], w[1], 2);
            *reinterpret_cast<u32x4*>(d + swz(row, 4 * part + 3)) = codes8(w[2], w[3], 2);
        }
    };
    auto qcommit = [&](int set, char* kd, char* vd, float* ksd, float* vsd) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < kQChunks; ++j) {
            const int c = kAttThreads * j + static_cast<int>(threadIdx.x);
            put_codes(kd, kc[set][j], c);           // codes, exact
            put_codes(vd, vc[set][j], c);
        }
        if (threadIdx.x < kUnit) {
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                ksd[b * kUnit + threadIdx.x] = kscl[set][b];
                vsd[b * kUnit + threadIdx.x] = vscl[set][b];
            }
        }
    };
    const float* ks_cur = kscl_s[0];           // scales of the unit being computed (quantized K, V)
    // 4-bit codes enter as c + kQBias (c = n - 8): a score slice is
    // scale * (K'Q - kQBias * sum of the slice's query values), the output
    // O - kQBias * (sum of the applied probabilities of the dim block)
    constexpr float kQBias = 136.f;
    float qsum[4] = {0.f, 0.f, 0.f, 0.f};     // head l16, dims 32 ks .. 32 ks + 31
    float psum[4] = {0.f, 0.f, 0.f, 0.f};     // head l16, dim block b: this lane's applied probabilities
    if constexpr (kQ == 2) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            float t = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) t += static_cast<float>(qb[ks][j]);
            qsum[ks] = kQBias * sum_xor32(sum_xor16(t));
        }
    }
    const float* vs_cur = vscl_s[0];

    float m_run = -INFINITY, l_run = 0.f;
    f32x4 acc[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // lane offsets: K rows 32w + 16t + l16; V rows 32w + 4*l4 + l16/4 (+16)
    int koff[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) koff[ks] = swz(32 * wave + l16, 4 * ks + l4);

    // Online-softmax update with keys 32w .. 32w+31 of unit u.  The unit's
    // K and V operands are read first; `release` runs once they are in
    // registers (the ring buffer may then be refilled) and before the math.
    auto compute = [&](int u, const char* kb, const char* vb, auto&& release) __attribute__((always_inline)) {
        // validity of this lane's keys 32w + 16t + 4*l4 + r
        uint32_t valid = 0;
        if (u < n_units)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = 32 * wave + 16 * t + 4 * l4 + r;
                const int tok = kTokenIds ? sel_s[u * kUnit + key] : sel_s[u] * kBlock + key;
                if (tok >= 0 && tok <= p) valid |= 1u << (4 * t + r);
            }
        const bool any = __builtin_amdgcn_ballot_w64(valid != 0) != 0;   // wave-uniform
        // K operands (lane: keys 32w + 16t + l16) and V^T operands
        bf16x8 kA[2][4];
        bf16x8 va[8];
        if (any) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    kA[t][ks] = *reinterpret_cast<const bf16x8*>(kb + 16 * t * kRowBytes + koff[ks]);
            // dim tile dt: keys 32w + 4*l4 + 0..3 and 32w + 16 + 4*l4 + 0..3
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                const int vo = swz(4 * l4 + (l16 >> 2), 2 * dt + ((l16 & 3) >> 1)) + (l16 & 1) * 8;
                const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(v4i16, vb + 32 * wave * kRowBytes + vo));
                const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    LDS_PTR(v4i16, vb + (32 * wave + 16) * kRowBytes + vo));
                va[dt] = __builtin_shufflevector(__builtin_bit_cast(bf16x4_t, lo), __builtin_bit_cast(bf16x4_t, hi),
                                                 0, 1, 2, 3, 4, 5, 6, 7);
            }
        }
        // S^T = K Q^T; lane gets keys 32w + 16t + 4*l4 + r of head l16
        f32x4 st[2];
        f32x4 vsc[kQ ? 4 : 1][2];                  // quantized V: scale of block b for this lane's keys
        if constexpr (kQ != 0) {
            // quantized K: slice ks is scale block ks of every key row, so each
            // slice's product is scaled per key; done before the release,
            // since the scales live in the ring unit's LDS
            if (any) {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    st[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) {
                        const f32x4 part = mfma_16x16x32_bf16(kA[t][ks], qb[ks], f32x4{0.f, 0.f, 0.f, 0.f});
                        const f32x4 sc = *reinterpret_cast<const f32x4*>(ks_cur + ks * kUnit + 32 * wave + 16 * t + 4 * l4);
                        if constexpr (kQ == 2) st[t] += sc * (part - qsum[ks]);
                        else st[t] += sc * part;
                    }
                }
#pragma unroll
                for (int b = 0; b < 4; ++b)
#pragma unroll
                    for (int t = 0; t < 2; ++t)
                        vsc[b][t] = *reinterpret_cast<const f32x4*>(vs_cur + b * kUnit + 32 * wave + 16 * t + 4 * l4);
            }
        }
        release();
        if (!any) return;                          // nothing of this wave's keys is visible
        if constexpr (kQ == 0) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                st[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) st[t] = mfma_16x16x32_bf16(kA[t][ks], qb[ks], st[t]);
            }
        }
        float x[8];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                x[4 * t + r] = ((valid >> (4 * t + r)) & 1) ? st[t][r] * qk_scale : -INFINITY;
        float cm = x[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) cm = fmaxf(cm, x[j]);
        cm = max_xor32(max_xor16(cm));
        const float m_new = fmaxf(m_run, cm);      // finite: the wave has a visible key
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 on the first unit
        float pr[8];
        float rs = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            pr[j] = __builtin_amdgcn_exp2f(x[j] - m_new);
            rs += pr[j];
        }
        rs = sum_xor32(sum_xor16(rs));
        l_run = l_run * alpha + rs;
        m_run = m_new;
        // P^T operand (B: k = key, n = head); k-slot 8*l4 + j holds key
        // 4*l4 + j (j < 4) or 16 + 4*l4 + (j - 4) of this wave's 32
        if constexpr (kQ == 0) {
            u32x4 pw;
            pw[0] = pack_bf16x2(pr[0], pr[1]);
            pw[1] = pack_bf16x2(pr[2], pr[3]);
            pw[2] = pack_bf16x2(pr[4], pr[5]);
            pw[3] = pack_bf16x2(pr[6], pr[7]);
            const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
            // O^T += V^T P^T
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) acc[dt] = mfma_16x16x32_bf16(va[dt], pb, acc[dt] * alpha);
        } else {
            // dims 32b .. 32b + 31 (tiles 2b, 2b + 1): P scaled by V's block-b scale per key
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                u32x4 pw;
                pw[0] = pack_bf16x2(pr[0] * vsc[b][0][0], pr[1] * vsc[b][0][1]);
                pw[1] = pack_bf16x2(pr[2] * vsc[b][0][2], pr[3] * vsc[b][0][3]);
                pw[2] = pack_bf16x2(pr[4] * vsc[b][1][0], pr[5] * vsc[b][1][1]);
                pw[3] = pack_bf16x2(pr[6] * vsc[b][1][2], pr[7] * vsc[b][1][3]);
                const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
                for (int dt = 2 * b; dt < 2 * b + 2; ++dt) acc[dt] = mfma_16x16x32_bf16(va[dt], pb, acc[dt] * alpha);
                if constexpr (kQ == 2) {
                    // this lane's 8 of the probabilities the product applied, rescaled
                    // as the accumulators are (the bias is subtracted after the loop)
                    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
                    const bf16x2_t ones2 = __builtin_bit_cast(bf16x2_t, 0x3F803F80u);   // {1, 1}
                    float ps = 0.f;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t wj = pw[j];
                        ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, wj), ones2, ps, false);
                    }
                    psum[b] = psum[b] * alpha + ps;
                }
            }
        }
    };

    // Two-unit ring: unit u + 1 streams in while unit u is computed.  Every
    // thread issues 2 * kCopiesPerUnit copies per unit, so waiting until at
    // most that many are outstanding means unit u has landed.  Only copies
    // into LDS are in flight in the loop.
    static_assert(kMaxUnits == 1 || kMaxUnits % 2 == 0, "units alternate between the two ring buffers");
    if constexpr (kQ == 0) {
        stage(0, kbuf0, vbuf0);
        if constexpr (kMaxUnits > 1) stage(1, kbuf1, vbuf1);
        auto step = [&](int u, const char* kb, const char* vb, char* kn, char* vn) __attribute__((always_inline)) {
            if (u + 1 < kMaxUnits) __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * kCopiesPerUnit));   // compile-time
            else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
            lds_barrier();                         // unit u is in LDS
            compute(u, kb, vb, [&]() __attribute__((always_inline)) {
                lds_barrier();                     // every wave has its operands: refill the buffers
                if (u + 2 < kMaxUnits) stage(u + 2, kn, vn);
            });
        };
#pragma unroll
        for (int u = 0; u < kMaxUnits; u += 2) {
            step(u, kbuf0, vbuf0, kbuf0, vbuf0);
            if constexpr (kMaxUnits > 1) step(u + 1, kbuf1, vbuf1, kbuf1, vbuf1);
        }
    } else {
        // quantized: unit u + 2 loads into register set u % 2 once every wave
        // holds unit u's operands; unit u + 1 (loaded one unit earlier) is
        // written to its buffer, freed at the release of unit u - 1, after the
        // math of unit u
        static_assert(kMaxUnits % 2 == 0, "the quantized ring is instantiated for even unit counts");
        qload(0, 0);
        qcommit(0, kbuf0, vbuf0, kscl_s[0], vscl_s[0]);
        qload(1, 1);
        auto qstep = [&](int u, int set, const char* kb, const char* vb, char* kn, char* vn, float* ksn,
                         float* vsn) __attribute__((always_inline)) {
            ks_cur = kscl_s[set];
            vs_cur = vscl_s[set];
            lds_barrier();                         // unit u is in LDS (written by every wave)
            compute(u, kb, vb, [&]() __attribute__((always_inline)) {
                lds_barrier();                     // every wave has its operands and scales
                if (u + 2 < kMaxUnits) qload(u + 2, set);
            });
            if (u + 1 < kMaxUnits) qcommit(set ^ 1, kn, vn, ksn, vsn);
        };
#pragma unroll
        for (int u = 0; u < kMaxUnits; u += 2) {
            qstep(u, 0, kbuf0, vbuf0, kbuf1, vbuf1, kscl_s[1], vscl_s[1]);
            qstep(u + 1, 1, kbuf1, vbuf1, kbuf0, vbuf0, kscl_s[0], vscl_s[0]);
        }
    }

    if constexpr (kQ == 2) {
        // the 4-bit codes' bias: kQBias times the applied probabilities of head l16
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const float vb = kQBias * sum_xor32(sum_xor16(psum[b]));
            acc[2 * b] -= f32x4{vb, vb, vb, vb};
            acc[2 * b + 1] -= f32x4{vb, vb, vb, vb};
        }
    }
    // ---- merge the four waves (lane holds O^T[dim 16*dt + 4*l4 + r][head l16])
    __syncthreads();
    float* mrg = reinterpret_cast<float*>(kbuf0);  // [wave][head][dim]
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
        *reinterpret_cast<f32x4*>(&mrg[(wave * kHeadsPerGroup + l16) * kHeadDim + 16 * dt + 4 * l4]) = acc[dt];
    if (lane < 16) {
        mrg_m[wave][lane] = m_run;
        mrg_l[wave][lane] = l_run;
    }
    __syncthreads();
    const int hh = threadIdx.x >> 4;          // head of this thread
    const int d0 = 8 * (threadIdx.x & 15);    // its 8 dims
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAttWaves; ++w) M = fmaxf(M, mrg_m[w][hh]);
    float L = 0.f;
    float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kAttWaves; ++w) {
        const float mw = mrg_m[w][hh];
        const float wt = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
        L += wt * mrg_l[w][hh];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] += wt * mrg[(w * kHeadsPerGroup + hh) * kHeadDim + d0 + e];
    }
    if (ka.n_split == 1) {
        const float inv = 1.f / L;
        float* dst = a.out + (i * kGroups * kHeadsPerGroup + g * kHeadsPerGroup + hh) * kHeadDim + d0;
        *reinterpret_cast<f32x4*>(dst) = f32x4{o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
        *reinterpret_cast<f32x4*>(dst + 4) = f32x4{o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv};
    } else if (a.arrive == nullptr) {
        float* part = static_cast<float*>(a.ws) + ((i * kGroups + g) * ka.n_split + sp) * kPartFloats;
        float* dst = part + hh * kHeadDim + d0;
        *reinterpret_cast<f32x4*>(dst) = f32x4{o[0], o[1], o[2], o[3]};
        *reinterpret_cast<f32x4*>(dst + 4) = f32x4{o[4], o[5], o[6], o[7]};
        if ((threadIdx.x & 15) == 0) {
            part[kHeadsPerGroup * kHeadDim + 2 * hh] = M;
            part[kHeadsPerGroup * kHeadDim + 2 * hh + 1] = L;
        }
    } else {
        // Decode step: the last split of this (query, group) to finish
        // merges the partials as the combine kernels do (split order,
        // against the largest m).  The partials of the pair are written and
        // read with system-coherent (sc1) buffer accesses, which go to and
        // come from memory past every XCD's L2, so they need no L2
        // write-back or invalidation: each thread waits for its partial
        // stores to complete before the barrier that precedes the arrival
        // (an agent-scope atomic), and the merging workgroup reads only
        // after the arrival returned.
        const int64_t pair = i * kGroups + g;
        const uint32_t pbytes = static_cast<uint32_t>(ka.n_split * kPartFloats * sizeof(float));
        const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
            static_cast<float*>(a.ws) + pair * ka.n_split * kPartFloats, 0, pbytes, 0x00020000);
        constexpr int kSc1 = 16;                  // cache policy: sc1
        constexpr int kMl = kHeadsPerGroup * kHeadDim;   // (m, l) of head h at kMl + 2h
        const int own = sp * kPartFloats;         // this split's partial, in floats
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{o[0], o[1], o[2], o[3]}), prs,
                                               4 * (own + hh * kHeadDim + d0), 0, kSc1);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{o[4], o[5], o[6], o[7]}), prs,
                                               4 * (own + hh * kHeadDim + d0 + 4), 0, kSc1);
        if ((threadIdx.x & 15) == 0) {
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(M), prs, 4 * (own + kMl + 2 * hh), 0, kSc1);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(L), prs, 4 * (own + kMl + 2 * hh + 1), 0, kSc1);
        }
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));     // this thread's partial stores have completed
        __shared__ int last_s;
        __syncthreads();
        if (threadIdx.x == 0)
            last_s = __hip_atomic_fetch_add(a.arrive + pair, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                     ka.n_split - 1;
        __syncthreads();
        if (last_s) {
            // the partials in batches of 16 splits, each batch's loads in
            // flight together (masked past the last split, whose weight is 0)
            constexpr int kB = 16;
            float Mx = -INFINITY;
            for (int s0 = 0; s0 < ka.n_split; s0 += kB) {
                float ms[kB];
#pragma unroll
                for (int j = 0; j < kB; ++j) {
                    const int jj = s0 + j < ka.n_split ? s0 + j : s0;
                    ms[j] = __uint_as_float(
                        __builtin_amdgcn_raw_buffer_load_b32(prs, 4 * (jj * kPartFloats + kMl + 2 * hh), 0, kSc1));
                }
#pragma unroll
                for (int j = 0; j < kB; ++j) Mx = fmaxf(Mx, s0 + j < ka.n_split ? ms[j] : -INFINITY);
            }
            float Lx = 0.f;
            float ox[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            for (int s0 = 0; s0 < ka.n_split; s0 += kB) {
                float ms[kB], ls[kB];
                f32x4 a0[kB], a1[kB];
#pragma unroll
                for (int j = 0; j < kB; ++j) {
                    const int jj = s0 + j < ka.n_split ? s0 + j : s0;
                    const int base = jj * kPartFloats;
                    ms[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(prs, 4 * (base + kMl + 2 * hh), 0, kSc1));
                    ls[j] = __uint_as_float(
                        __builtin_amdgcn_raw_buffer_load_b32(prs, 4 * (base + kMl + 2 * hh + 1), 0, kSc1));
                    a0[j] = __builtin_bit_cast(
                        f32x4, __builtin_amdgcn_raw_buffer_load_b128(prs, 4 * (base + hh * kHeadDim + d0), 0, kSc1));
                    a1[j] = __builtin_bit_cast(
                        f32x4, __builtin_amdgcn_raw_buffer_load_b128(prs, 4 * (base + hh * kHeadDim + d0 + 4), 0, kSc1));
                }
#pragma unroll
                for (int j = 0; j < kB; ++j) {                   // in split order
                    const float mj = s0 + j < ka.n_split ? ms[j] : -INFINITY;
                    const float wt = (mj == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mj - Mx);
                    Lx += wt * ls[j];
                    ox[0] += wt * a0[j].x; ox[1] += wt * a0[j].y; ox[2] += wt * a0[j].z; ox[3] += wt * a0[j].w;
                    ox[4] += wt * a1[j].x; ox[5] += wt * a1[j].y; ox[6] += wt * a1[j].z; ox[7] += wt * a1[j].w;
                }
            }
            const float inv = 1.f / Lx;
            float* od = a.out + (i * kGroups * kHeadsPerGroup + g * kHeadsPerGroup + hh) * kHeadDim + d0;
            *reinterpret_cast<f32x4*>(od) = f32x4{ox[0] * inv, ox[1] * inv, ox[2] * inv, ox[3] * inv};
            *reinterpret_cast<f32x4*>(od + 4) = f32x4{ox[4] * inv, ox[5] * inv, ox[6] * inv, ox[7] * inv};
        }
    }
}

// Fixed-order merge of the split partials of one (query, group), in one
// pass: a thread owns 8 dims of one head and loads the (m, l, acc) of all
// kNs splits at once (one round trip to memory), then combines them in
// split order against their largest m.
template <int kNs>
__global__ __launch_bounds__(256) void attend_combine_kernel(const float* __restrict__ ws, float* __restrict__ out) {
    const int g = static_cast<int>(blockIdx.x % kGroups);
    const int64_t i = blockIdx.x / kGroups;
    const int hh = threadIdx.x >> 4;
    const int d0 = 8 * (threadIdx.x & 15);
    const float* part0 = ws + (i * kGroups + g) * kNs * static_cast<int64_t>(kPartFloats);
    constexpr int kMl = kHeadsPerGroup * kHeadDim;   // (m, l) of head h at kMl + 2h
    float ms[kNs], ls[kNs];
    f32x4 a0[kNs], a1[kNs];
#pragma unroll
    for (int j = 0; j < kNs; ++j) {
        const float* part = part0 + j * kPartFloats;
        ms[j] = part[kMl + 2 * hh];
        ls[j] = part[kMl + 2 * hh + 1];
        a0[j] = *reinterpret_cast<const f32x4*>(part + hh * kHeadDim + d0);
        a1[j] = *reinterpret_cast<const f32x4*>(part + hh * kHeadDim + d0 + 4);
    }
    float M = -INFINITY;
#pragma unroll
    for (int j = 0; j < kNs; ++j) M = fmaxf(M, ms[j]);
    float L = 0.f;
    float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kNs; ++j) {                  // in split order
        const float wt = (ms[j] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ms[j] - M);
        L += wt * ls[j];
        o[0] += wt * a0[j].x; o[1] += wt * a0[j].y; o[2] += wt * a0[j].z; o[3] += wt * a0[j].w;
        o[4] += wt * a1[j].x; o[5] += wt * a1[j].y; o[6] += wt * a1[j].z; o[7] += wt * a1[j].w;
    }
    const float inv = 1.f / L;
    float* dst = out + (i * kGroups * kHeadsPerGroup + g * kHeadsPerGroup + hh) * kHeadDim + d0;
    *reinterpret_cast<f32x4*>(dst) = f32x4{o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
    *reinterpret_cast<f32x4*>(dst + 4) = f32x4{o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv};
}

// The same merge for any number of splits (more than 16: one query over many
// blocks); the partials of up to kCombineBatch splits are loaded together
// (one round trip to memory per batch, not per split).
constexpr int kCombineBatch = 16;

__global__ __launch_bounds__(256) void attend_combine_any_kernel(const float* __restrict__ ws,
                                                             int n_split, float* __restrict__ out) {
    const int g = static_cast<int>(blockIdx.x % kGroups);
    const int64_t i = blockIdx.x / kGroups;
    const int hh = threadIdx.x >> 4;
    const int d0 = 8 * (threadIdx.x & 15);
    const float* part0 = ws + (i * kGroups + g) * n_split * static_cast<int64_t>(kPartFloats);
    constexpr int kMl = kHeadsPerGroup * kHeadDim;   // (m, l) of head h at kMl + 2h
    float M = -INFINITY;
    for (int s0 = 0; s0 < n_split; s0 += kCombineBatch) {
        float ms[kCombineBatch];
#pragma unroll
        for (int j = 0; j < kCombineBatch; ++j)
            ms[j] = s0 + j < n_split ? part0[(s0 + j) * kPartFloats + kMl + 2 * hh] : -INFINITY;
#pragma unroll
        for (int j = 0; j < kCombineBatch; ++j) M = fmaxf(M, ms[j]);
    }
    float L = 0.f;
    float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < n_split; s0 += kCombineBatch) {
        float ms[kCombineBatch], ls[kCombineBatch];
        f32x4 a0[kCombineBatch], a1[kCombineBatch];
#pragma unroll
        for (int j = 0; j < kCombineBatch; ++j) {
            const float* part = part0 + (s0 + j < n_split ? s0 + j : s0) * kPartFloats;
            ms[j] = s0 + j < n_split ? part[kMl + 2 * hh] : -INFINITY;
            ls[j] = part[kMl + 2 * hh + 1];
            a0[j] = *reinterpret_cast<const f32x4*>(part + hh * kHeadDim + d0);
            a1[j] = *reinterpret_cast<const f32x4*>(part + hh * kHeadDim + d0 + 4);
        }
#pragma unroll
        for (int j = 0; j < kCombineBatch; ++j) {      // in split order
            const float wt = (ms[j] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ms[j] - M);
            L += wt * ls[j];
            o[0] += wt * a0[j].x; o[1] += wt * a0[j].y; o[2] += wt * a0[j].z; o[3] += wt * a0[j].w;
            o[4] += wt * a1[j].x; o[5] += wt * a1[j].y; o[6] += wt * a1[j].z; o[7] += wt * a1[j].w;
        }
    }
    const float inv = 1.f / L;
    float* dst = out + (i * kGroups * kHeadsPerGroup + g * kHeadsPerGroup + hh) * kHeadDim + d0;
    *reinterpret_cast<f32x4*>(dst) = f32x4{o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
    *reinterpret_cast<f32x4*>(dst + 4) = f32x4{o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv};
}

int num_units(int sel_len, int unit) {
    return unit == kBlock ? sel_len : (sel_len + kUnit - 1) / kUnit;
}

constexpr int kUnitsPerSplitMax = 8;
static_assert(kMaxSplitEntries == kUnitsPerSplitMax * kUnit, "ids one split stages");

// instantiations for splits of up to 2, 4 and 8 units
template <int kQ>
void launch_units(const KernelArgs& ka, bool blocks, int nu, dim3 grid, hipStream_t s) {
    if (blocks) {
        if (nu == 1 && kQ == 0) hipLaunchKernelGGL((attend_kernel<false, 1, 0>), grid, dim3(kAttThreads), 0, s, ka);
        else if (nu <= 2) hipLaunchKernelGGL((attend_kernel<false, 2, kQ>), grid, dim3(kAttThreads), 0, s, ka);
        else if (nu <= 4) hipLaunchKernelGGL((attend_kernel<false, 4, kQ>), grid, dim3(kAttThreads), 0, s, ka);
        else hipLaunchKernelGGL((attend_kernel<false, kUnitsPerSplitMax, kQ>), grid, dim3(kAttThreads), 0, s, ka);
    } else {
        if (nu == 1 && kQ == 0) hipLaunchKernelGGL((attend_kernel<true, 1, 0>), grid, dim3(kAttThreads), 0, s, ka);
        else if (nu <= 2) hipLaunchKernelGGL((attend_kernel<true, 2, kQ>), grid, dim3(kAttThreads), 0, s, ka);
        else if (nu <= 4) hipLaunchKernelGGL((attend_kernel<true, 4, kQ>), grid, dim3(kAttThreads), 0, s, ka);
        else hipLaunchKernelGGL((attend_kernel<true, kUnitsPerSplitMax, kQ>), grid, dim3(kAttThreads), 0, s, ka);
    }
}

}  // namespace

int attend_num_splits(int64_t n_q, int sel_len, int unit) {
    const int64_t pairs = n_q * kGroups;
    if (pairs <= 0) return 1;   // an empty call: nothing is split
    const int n_units = num_units(sel_len, unit);
    // about one workgroup per compute unit (256), each streaming >= 1 unit,
    // and at most kUnitsPerSplitMax units per split
    int64_t want = (256 + pairs - 1) / pairs;
    if (want > n_units) want = n_units;
    const int64_t least = (n_units + kUnitsPerSplitMax - 1) / kUnitsPerSplitMax;
    if (want < least) want = least;
    if (want < 1) want = 1;
    return static_cast<int>(want);
}

size_t attend_ws_bytes(int64_t n_q, int sel_len, int unit) {
    if (n_q <= 0) return 0;
    const int n_split = attend_num_splits(n_q, sel_len, unit);
    if (n_split == 1) return 0;
    return static_cast<size_t>(n_q) * kGroups * n_split * kPartFloats * sizeof(float);
}

hipError_t launch_attend(const AttendArgs& a, hipStream_t s) {
    KernelArgs ka;
    ka.a = a;
    ka.n_split = attend_num_splits(a.n_q, a.sel_len, a.unit);
    ka.n_units = num_units(a.sel_len, a.unit);
    ka.units_per_split = (ka.n_units + ka.n_split - 1) / ka.n_split;
    const dim3 grid(static_cast<unsigned>(a.n_q * kGroups * ka.n_split));
    const int nu = ka.units_per_split;
    switch (a.kv_format) {
        case 0: launch_units<0>(ka, a.unit == kBlock, nu, grid, s); break;
        case 1: launch_units<1>(ka, a.unit == kBlock, nu, grid, s); break;
        case 2: launch_units<2>(ka, a.unit == kBlock, nu, grid, s); break;
        default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || ka.n_split == 1 || a.arrive != nullptr) return e;   // (arrival: merged in the kernel)
    const dim3 cgrid(static_cast<unsigned>(a.n_q * kGroups));
    const float* part = static_cast<const float*>(a.ws);
    switch (ka.n_split) {
#define MSA_COMBINE_CASE(N) case N: hipLaunchKernelGGL(attend_combine_kernel<N>, cgrid, dim3(256), 0, s, part, a.out); break;
        MSA_COMBINE_CASE(2) MSA_COMBINE_CASE(3) MSA_COMBINE_CASE(4) MSA_COMBINE_CASE(5) MSA_COMBINE_CASE(6)
        MSA_COMBINE_CASE(7) MSA_COMBINE_CASE(8) MSA_COMBINE_CASE(9) MSA_COMBINE_CASE(10) MSA_COMBINE_CASE(11)
        MSA_COMBINE_CASE(12) MSA_COMBINE_CASE(13) MSA_COMBINE_CASE(14) MSA_COMBINE_CASE(15) MSA_COMBINE_CASE(16)
#undef MSA_COMBINE_CASE
        default: hipLaunchKernelGGL(attend_combine_any_kernel, cgrid, dim3(256), 0, s, part, ka.n_split, a.out);
    }
    return hipGetLastError();
}

}  // namespace msa
