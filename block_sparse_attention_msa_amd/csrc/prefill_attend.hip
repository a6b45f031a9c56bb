// prefill_attend.hip -- block-sparse attention for a prefill chunk.
//
// "Add MiniMax-M3 (MSA: MiniMax Sparse Attention) support", Implementation,
// batch path: each query attends only over its group's selected blocks
// (causal inside the query's own block); prefill and decode rank the same
// block scores, so the selection semantics are those of decode.
//
// Design (gfx950).  A workgroup takes a tile of 16 consecutive queries of one
// group and sweeps the UNION of their selected blocks in ascending block
// order.  Each block's K and V (128 keys x 256 B each) are copied straight
// from HBM into LDS with global_load_lds_dwordx4 -- no registers -- into one
// of two buffers, so the next block streams in while the current one is
// consumed by every query of the tile that selected it.  Rows are stored
// with their 16-byte segments permuted by the row index, so the K operand
// reads (16 rows, same columns) and the V reads are free of bank conflicts.
// V stays row-major: ds_read_b64_tr_b16 hands each lane four consecutive keys
// of one dim, which is the layout the P.V matrix-core operand wants.  Eight
// waves each own two queries; their online-softmax states and 16-head x
// 128-dim accumulators stay in registers for the whole sweep.
#include "common.hpp"

namespace msa {
namespace {

constexpr int kPaWaves = 8;
constexpr int kSlots = 2;                   // queries per wave
constexpr int kTileQ = kSlots * kPaWaves;   // queries per workgroup
constexpr int kPaThreads = 64 * kPaWaves;
constexpr int kRowBytes = kHeadDim * 2;     // one group's K or V row: 256 B = 16 segments
constexpr int kBufBytes = kBlock * kRowBytes;   // 32 KiB per block for K (and for V)
constexpr int kStageSlots = kBlock * kRowBytes / 16 / kPaWaves;   // 16-byte slots per wave and operand
constexpr float kLog2eP = 1.4426950408889634f;
constexpr int kRing = 3;                    // operand register ring depth (steps)
constexpr float kSlack = 8.f;              // lazy-rescale threshold, log2 units

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

// Rows are stored with their 16 segments permuted by seg ^ f(row & 15), f a
// 4-bit rotate: f is one-to-one on 16 consecutive rows (the K operand reads
// 16 rows at one segment) and f >> 1 is one-to-one on 8 consecutive rows (the
// transposing V reads take a 32-byte pair of segments from each of 8 rows per
// half-wave), so neither read pattern has bank conflicts.
__device__ __forceinline__ int rowperm(int row) { return ((row & 7) << 1) | ((row >> 3) & 1); }
// Byte offset of 16-byte segment `seg` of row `row` in a staged buffer.
__device__ __forceinline__ int swz(int row, int seg) { return row * kRowBytes + ((seg ^ rowperm(row)) << 4); }

__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), bf16x2_t));
}
struct PaArgs {
    const uint16_t* k;
    const uint16_t* v;
    int64_t cap;
    const uint16_t* q;
    int32_t stream;
    int32_t pos0;
    int64_t n_q;
    int64_t last_row;
    const int32_t* sel;
    int top_k;
    int nblk;
    int n_tiles;
    float scale;
    float* out;
};

__global__ __launch_bounds__(kPaThreads, 1) void prefill_attend_kernel(PaArgs a) {
    // workgroup id -> (group, tile); with 8 XCDs fed round-robin, each XCD
    // serves one group
    const int g = blockIdx.x % kGroups;
    const int tile = blockIdx.x / kGroups;
    if (tile >= a.n_tiles) return;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l16 = lane & 15;
    const int l4 = lane >> 4;
    const int64_t q_first = static_cast<int64_t>(tile) * kTileQ;
    const int n_tq = static_cast<int>(min<int64_t>(kTileQ, a.n_q - q_first));

    // two staging buffers, each K then V of one block; separate objects so
    // the compiler can tell reads of one from the loads into the other
    __shared__ __attribute__((aligned(16))) char kv0[2][kBufBytes];
    __shared__ __attribute__((aligned(16))) char kv1[2][kBufBytes];
    __shared__ int wave_sums[kPaWaves];
    __shared__ int s_nu;
    extern __shared__ uint32_t dyn[];          // qmask[nblk], then ulist[nblk] (16-bit ids)
    uint32_t* qmask = dyn;
    uint16_t* ulist = reinterpret_cast<uint16_t*>(dyn + a.nblk);

    // ---- which tile queries selected which block
    for (int b = threadIdx.x; b < a.nblk; b += kPaThreads) qmask[b] = 0u;
    __syncthreads();
    for (int e = threadIdx.x; e < n_tq * a.top_k; e += kPaThreads) {
        const int t = e / a.top_k;
        const int64_t qi = q_first + t;
        const int blk = a.sel[(qi * kGroups + g) * a.top_k + e % a.top_k];
        const int loc = (a.pos0 + static_cast<int>(qi)) / kBlock;
        if (blk >= 0 && blk <= loc) atomicOr(&qmask[blk], 1u << t);
    }
    __syncthreads();
    // ---- compact the union in ascending block order
    {
        const int per = (a.nblk + kPaThreads - 1) / kPaThreads;
        const int b0 = threadIdx.x * per, b1 = min(b0 + per, a.nblk);
        int cnt = 0;
        for (int b = b0; b < b1; ++b) cnt += qmask[b] != 0u;
        int incl = cnt;                        // inclusive scan over the workgroup
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
        for (int b = b0; b < b1; ++b)
            if (qmask[b] != 0u) ulist[pos++] = static_cast<uint16_t>(b);
        if (threadIdx.x == kPaThreads - 1) s_nu = before + incl;
        __syncthreads();
    }
    const int n_union = s_nu;

    // ---- per-slot query state: wave owns tile queries kSlots * wave + s
    const int64_t s_base = static_cast<int64_t>(a.stream) * a.cap * kGroups;
    bf16x8 qb[kSlots][4];
    f32x4 acc[kSlots][8];
    float m_run[kSlots], l_run[kSlots];
    int pq[kSlots];
#pragma unroll
    for (int s = 0; s < kSlots; ++s) {
        const int t = kSlots * wave + s;
        const int64_t qi = min<int64_t>(q_first + t, a.n_q - 1);
        pq[s] = a.pos0 + static_cast<int>(q_first + t);
        const uint16_t* qrow = a.q + (qi * kGroups * kHeadsPerGroup + g * kHeadsPerGroup + l16) * kHeadDim;
#pragma unroll
        for (int ks4 = 0; ks4 < 4; ++ks4) qb[s][ks4] = *reinterpret_cast<const bf16x8*>(qrow + 32 * ks4 + 8 * l4);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) acc[s][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        m_run[s] = -INFINITY;
        l_run[s] = 0.f;
    }
    const float qk_scale = a.scale * kLog2eP;

    // Lane offsets of the operand reads inside a staged buffer.  The row
    // permutation depends on row & 15 only, so chunk and tile offsets (whole
    // multiples of 16 rows) are added as constants.
    int koff[4];                                  // K: row l16, segment 4*ks4 + l4
#pragma unroll
    for (int ks4 = 0; ks4 < 4; ++ks4) koff[ks4] = swz(l16, 4 * ks4 + l4);
    int voff[8];                                  // V: row 4*l4 + l16/4, dims 16*dt + 4*(l16%4)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) voff[dt] = swz(4 * l4 + (l16 >> 2), 2 * dt + ((l16 & 3) >> 1)) + (l16 & 1) * 8;

    // Direct-to-LDS staging of block b into `dst` (K, then V): 2048 16-byte
    // slots each; the wave's instruction j fills slots kStageSlots * wave +
    // 64 * j + lane, i.e. row slot / 16 at permuted position slot % 16, which
    // receives the row's segment (slot % 16) ^ f(row).
    uint32_t soff[kStageSlots / 64];              // lane's source offset (elements) within a block
#pragma unroll
    for (int j = 0; j < kStageSlots / 64; ++j) {
        const int slot = kStageSlots * wave + 64 * j + lane;
        const int row = slot >> 4;
        soff[j] = static_cast<uint32_t>(row * kGroups * kHeadDim + 8 * ((slot & 15) ^ rowperm(row)));
    }
    auto stage = [&](int b, char (*dst)[kBufBytes]) {
        const int64_t row0 = static_cast<int64_t>(b) * kBlock;
        const int64_t base = (s_base + row0 * kGroups + g) * kHeadDim;
        const uint16_t* kbase = a.k + base;
        const uint16_t* vbase = a.v + base;
        if (row0 + kBlock - 1 <= a.last_row) {        // wave-uniform: the whole block is written
#pragma unroll
            for (int j = 0; j < kStageSlots / 64; ++j) {
                __builtin_amdgcn_global_load_lds(kbase + soff[j], LDS_PTR(void, &dst[0][(kStageSlots * wave + 64 * j) * 16]),
                                                 16, 0, 0);
                __builtin_amdgcn_global_load_lds(vbase + soff[j], LDS_PTR(void, &dst[1][(kStageSlots * wave + 64 * j) * 16]),
                                                 16, 0, 0);
            }
        } else {
            // rows past the chunk's last key are clamped to it: they are
            // masked for every query, and a written row keeps P.V finite
            const int last = static_cast<int>(a.last_row - row0);
#pragma unroll
            for (int j = 0; j < kStageSlots / 64; ++j) {
                const int row = (kStageSlots * wave + 64 * j + lane) >> 4;
                const uint32_t o = soff[j] - static_cast<uint32_t>((row - min(row, last)) * kGroups * kHeadDim);
                __builtin_amdgcn_global_load_lds(kbase + o, LDS_PTR(void, &dst[0][(kStageSlots * wave + 64 * j) * 16]),
                                                 16, 0, 0);
                __builtin_amdgcn_global_load_lds(vbase + o, LDS_PTR(void, &dst[1][(kStageSlots * wave + 64 * j) * 16]),
                                                 16, 0, 0);
            }
        }
    };

    // Consume the block staged in `src`: every tile query of this wave that
    // selected block b attends over its 128 keys with one softmax update.
    // Both products run as steps of four LDS reads and a few independent MFMAs;
    // reads are issued kRing - 1 steps ahead into a kRing-deep register ring,
    // so at most 4 * kRing are in flight (the LDS counter counts to 15) and
    // each step waits only for its own.  Scheduling barriers keep that order.
    auto consume = [&](int b, unsigned bmask, const char (*src)[kBufBytes]) {
        const unsigned my = (bmask >> (kSlots * wave)) & ((1u << kSlots) - 1);
        if (my == 0) return;                            // wave-uniform
        const char* kb = src[0];
        const char* vb = src[1];
        // S step i: 16-key tiles e = 4*(i&1) + t, dims 32*(i>>1) + 8*l4 ..
        auto load_ks = [&](int i, bf16x8 (&o)[4]) {
#pragma unroll
            for (int t = 0; t < 4; ++t)
                o[t] = *reinterpret_cast<const bf16x8*>(kb + 16 * (4 * (i & 1) + t) * kRowBytes + koff[i >> 1]);
        };
        // P.V step i: chunk c = i>>2, dim tiles dt = 2*(i&3) + u.  Transposing
        // reads: within each 16-lane row, lane j addresses row key0 + j/4,
        // dims d0 + 4*(j%4) .. +3, and receives V[key0 + 0..3][d0 + j], with
        // key0 = 32c + 4*l4 for k-slots 0..3 and 32c + 16 + 4*l4 for 4..7
        auto load_vs = [&](int i, bf16x8 (&o)[2]) {
            const int c = i >> 2;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int dt = 2 * (i & 3) + u;
                const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    LDS_PTR(v4i16, vb + kChunk * c * kRowBytes + voff[dt]));
                const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    LDS_PTR(v4i16, vb + (kChunk * c + 16) * kRowBytes + voff[dt]));
                o[u] = __builtin_shufflevector(__builtin_bit_cast(bf16x4_t, lo), __builtin_bit_cast(bf16x4_t, hi),
                                               0, 1, 2, 3, 4, 5, 6, 7);
            }
        };
#pragma unroll
        for (int s = 0; s < kSlots; ++s) {
            if (!((my >> s) & 1)) continue;             // wave-uniform
            const int kmax = pq[s] - b * kBlock;        // last visible key offset, >= 0
            // S^T = K Q^T: st[e] holds keys 16e + 4*l4 + r, head l16.  Keys
            // past the query are computed and then masked: every staged row
            // holds finite values.
            f32x4 st[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) st[e] = f32x4{0.f, 0.f, 0.f, 0.f};
            bf16x8 kr[kRing][4];
#pragma unroll
            for (int i = 0; i < kRing - 1; ++i) load_ks(i, kr[i]);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if (i + kRing - 1 < 8) load_ks(i + kRing - 1, kr[(i + kRing - 1) % kRing]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    st[4 * (i & 1) + t] = mfma_16x16x32_bf16(kr[i % kRing][t], qb[s][i >> 1], st[4 * (i & 1) + t]);
                __builtin_amdgcn_sched_barrier(0);
            }
            bf16x8 vr[kRing][2];
#pragma unroll
            for (int i = 0; i < kRing - 1; ++i) load_vs(i, vr[i]);
            // Mask keys past the query (only its own block has any), then the
            // block max of the raw scores; the scale is positive.
            if (kmax < kBlock - 1) {                    // wave-uniform
                const int rel = kmax - 4 * l4;          // compared with constants: no index registers
#pragma unroll
                for (int e = 0; e < 8; ++e)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (16 * e + r > rel) st[e][r] = -INFINITY;
            }
            float mx = st[0][0];
#pragma unroll
            for (int e = 0; e < 8; ++e)
#pragma unroll
                for (int r = 0; r < 4; ++r) mx = fmaxf(mx, st[e][r]);
            mx = max_xor32(max_xor16(mx)) * qk_scale;   // key 0 is visible: finite
            // Lazy rescaling: the reference max m_run moves only when a block
            // max exceeds it by more than kSlack (log2 units), so probabilities
            // stay below 2^kSlack and most blocks skip rescaling the
            // accumulators.  The result is the same softmax.
            if (__builtin_amdgcn_ballot_w64(mx > m_run[s] + kSlack) != 0) {   // wave-uniform
                const float m_new = fmaxf(m_run[s], mx);
                const float alpha = __builtin_amdgcn_exp2f(m_run[s] - m_new);   // 0 on the first block
                l_run[s] *= alpha;
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) acc[s][dt] = acc[s][dt] * alpha;
                m_run[s] = m_new;
            }
            // P^T as the B operand of P.V: k-slot 8*l4 + j of chunk c is key
            // 32c + 4*l4 + j (j < 4) or 32c + 16 + 4*l4 + j - 4 (j >= 4)
            bf16x8 pb[kBlock / kChunk];
            float rs = 0.f;
#pragma unroll
            for (int c = 0; c < kBlock / kChunk; ++c) {
                float pr[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    pr[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(st[2 * c + j / 4][j % 4], qk_scale, -m_run[s]));
                    rs += pr[j];
                }
                u32x4 pw;
                pw[0] = pack2_bf16(pr[0], pr[1]);
                pw[1] = pack2_bf16(pr[2], pr[3]);
                pw[2] = pack2_bf16(pr[4], pr[5]);
                pw[3] = pack2_bf16(pr[6], pr[7]);
                pb[c] = __builtin_bit_cast(bf16x8, pw);
            }
            l_run[s] += sum_xor32(sum_xor16(rs));
            // O^T += V^T P^T
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                if (i + kRing - 1 < 16) load_vs(i + kRing - 1, vr[(i + kRing - 1) % kRing]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int u = 0; u < 2; ++u)
                    acc[s][2 * (i & 3) + u] =
                        mfma_16x16x32_bf16(vr[i % kRing][u], pb[i >> 2], acc[s][2 * (i & 3) + u]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    // The block ids and masks are read before the loads are issued: LDS reads
    // that the compiler cannot tell apart from the staging buffers would
    // otherwise wait for the loads in flight.
    int b_cur = n_union > 0 ? static_cast<int>(ulist[0]) : 0;
    if (n_union > 0) stage(b_cur, kv0);
    for (int u = 0; u < n_union; u += 2) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        int b_next = u + 1 < n_union ? static_cast<int>(ulist[u + 1]) : 0;
        unsigned m_cur = qmask[b_cur];
        if (u + 1 < n_union) stage(b_next, kv1);
        consume(b_cur, m_cur, kv0);
        if (u + 1 >= n_union) break;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        b_cur = u + 2 < n_union ? static_cast<int>(ulist[u + 2]) : 0;
        m_cur = qmask[b_next];
        if (u + 2 < n_union) stage(b_cur, kv0);
        consume(b_next, m_cur, kv1);
    }

    // ---- normalise and write: lane holds O^T[dim 16*dt + 4*l4 + r][head l16]
#pragma unroll
    for (int s = 0; s < kSlots; ++s) {
        const int t = kSlots * wave + s;
        if (t >= n_tq) continue;
        const int64_t qi = q_first + t;
        const float inv = 1.f / l_run[s];
        float* dst = a.out + (qi * kGroups * kHeadsPerGroup + g * kHeadsPerGroup + l16) * kHeadDim + 4 * l4;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<f32x4*>(dst + 16 * dt) = acc[s][dt] * inv;
    }
}

}  // namespace

hipError_t launch_prefill_attend(const uint16_t* k, const uint16_t* v, int64_t cap, const uint16_t* q,
                                 int32_t stream, int32_t pos0, int64_t n_q, const int32_t* sel, int top_k,
                                 float scale, float* out, hipStream_t s) {
    PaArgs a;
    a.k = k;
    a.v = v;
    a.cap = cap;
    a.q = q;
    a.stream = stream;
    a.pos0 = pos0;
    a.n_q = n_q;
    a.last_row = pos0 + n_q - 1;
    a.sel = sel;
    a.top_k = top_k;
    a.nblk = (pos0 + static_cast<int>(n_q) - 1) / kBlock + 1;
    a.n_tiles = static_cast<int>((n_q + kTileQ - 1) / kTileQ);
    a.scale = scale;
    a.out = out;
    const unsigned n_wg = static_cast<unsigned>(a.n_tiles) * kGroups;
    const size_t lds = static_cast<size_t>(a.nblk) * (sizeof(uint32_t) + sizeof(uint16_t));
    hipLaunchKernelGGL(prefill_attend_kernel, dim3(n_wg), dim3(kPaThreads), lds, s, a);
    return hipGetLastError();
}

}  // namespace msa
