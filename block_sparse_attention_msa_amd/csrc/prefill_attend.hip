// prefill_attend.hip -- block-sparse attention for a prefill chunk.
//
// "Add MiniMax-M3 (MSA: MiniMax Sparse Attention) support", Implementation,
// batch path: each query attends only over its group's selected blocks
// (causal inside the query's own block); prefill and decode rank the same
// block scores, so the selection semantics are those of decode.
//
// Design (gfx950): the selections of neighbouring queries overlap only a
// little (about 16 of 256 blocks each, plus the shared local block), so a
// workgroup takes a tile of 24 consecutive queries of one group and sweeps the
// UNION of their selected blocks in ascending block order.  Each block's K
// (row-major) and V (transposed) are staged into LDS once and consumed by
// every query of the tile that selected it, which cuts the K/V traffic by the
// overlap factor.  Eight waves each own three queries; their online-softmax
// states and 16-head x 128-dim accumulators stay in registers for the whole
// sweep.  Workgroups are laid out so that the two XCDs sharing an id pair
// serve one group, so concurrently running tiles sweep the same blocks and
// their K/V is reused from L2.
#include "common.hpp"

namespace msa {
namespace {

constexpr int kTileQ = 24;                 // queries per workgroup
constexpr int kPaWaves = 8;
constexpr int kSlots = kTileQ / kPaWaves;  // queries per wave
constexpr int kPaThreads = 64 * kPaWaves;
constexpr int kPitch = kHeadDim + 8;       // bf16 per LDS row (K rows, V^T rows)
constexpr float kLog2eP = 1.4426950408889634f;

__device__ __forceinline__ float max_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
    const __bf16 a = static_cast<__bf16>(lo);
    const __bf16 b = static_cast<__bf16>(hi);
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, a)) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b)) << 16);
}

struct PaArgs {
    const uint16_t* k;
    const uint16_t* v;
    int64_t cap;
    const uint16_t* q;
    int32_t stream;
    int32_t pos0;
    int64_t n_q;
    const int32_t* sel;
    int top_k;
    int nblk;
    int n_tiles;
    float scale;
    float* out;
};

__global__ __launch_bounds__(kPaThreads, 2) void prefill_attend_kernel(PaArgs a) {
    // id -> (group, tile): ids 8j + 2g + h serve group g, tile 2j + h
    const int id = blockIdx.x;
    const int g = (id & 7) >> 1;
    const int tile = 2 * (id >> 3) + (id & 1);
    if (tile >= a.n_tiles) return;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int l16 = lane & 15;
    const int l4 = lane >> 4;
    const int64_t q_first = static_cast<int64_t>(tile) * kTileQ;
    const int n_tq = static_cast<int>(min<int64_t>(kTileQ, a.n_q - q_first));

    __shared__ uint16_t ks[kBlock * kPitch];      // K rows of the staged block
    __shared__ uint16_t vt[kHeadDim * kPitch];    // V^T of the staged block
    extern __shared__ unsigned long long qmask[]; // [nblk]: tile queries that selected each block

    // ---- which tile queries selected which block
    for (int b = threadIdx.x; b < a.nblk; b += kPaThreads) qmask[b] = 0ull;
    __syncthreads();
    for (int e = threadIdx.x; e < n_tq * a.top_k; e += kPaThreads) {
        const int t = e / a.top_k;
        const int64_t qi = q_first + t;
        const int blk = a.sel[(qi * kGroups + g) * a.top_k + e % a.top_k];
        const int loc = (a.pos0 + static_cast<int>(qi)) / kBlock;
        if (blk >= 0 && blk <= loc) atomicOr(&qmask[blk], 1ull << t);
    }
    __syncthreads();

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
    const int my_bits_shift = kSlots * wave;

    for (int b = 0; b < a.nblk; ++b) {
        const unsigned long long mask = qmask[b];       // uniform across the workgroup
        if (mask == 0ull) continue;
        // ---- stage K_b rows and V_b^T (rows past the cache are clamped; those
        // keys are past every query's position and masked)
        __syncthreads();                                // the previous block is consumed
        {
            const int64_t row0 = static_cast<int64_t>(b) * kBlock;
#pragma unroll
            for (int kpc = 0; kpc < 4; ++kpc) {          // K: 2048 pieces of 16 B, 4 per thread
                const int piece = threadIdx.x + kPaThreads * kpc;
                const int r = piece >> 4, seg = piece & 15;
                const int64_t row = min<int64_t>(row0 + r, a.cap - 1);
                const u32x4 x = *reinterpret_cast<const u32x4*>(a.k + (s_base + row * kGroups + g) * kHeadDim + 8 * seg);
                *reinterpret_cast<u32x4*>(&ks[r * kPitch + 8 * seg]) = x;
            }
            {                                           // V: one (4-key quad, 8-dim segment) per thread
                const int qd = threadIdx.x >> 4, seg = threadIdx.x & 15;
                u32x4 w[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int64_t row = min<int64_t>(row0 + 4 * qd + u, a.cap - 1);
                    w[u] = *reinterpret_cast<const u32x4*>(a.v + (s_base + row * kGroups + g) * kHeadDim + 8 * seg);
                }
#pragma unroll
                for (int m2 = 0; m2 < 4; ++m2) {
                    const uint32_t e01 = __builtin_amdgcn_perm(w[1][m2], w[0][m2], 0x05040100);
                    const uint32_t e23 = __builtin_amdgcn_perm(w[3][m2], w[2][m2], 0x05040100);
                    const uint32_t o01 = __builtin_amdgcn_perm(w[1][m2], w[0][m2], 0x07060302);
                    const uint32_t o23 = __builtin_amdgcn_perm(w[3][m2], w[2][m2], 0x07060302);
                    const int d = 8 * seg + 2 * m2;
                    *reinterpret_cast<uint2*>(&vt[d * kPitch + 4 * qd]) = make_uint2(e01, e23);
                    *reinterpret_cast<uint2*>(&vt[(d + 1) * kPitch + 4 * qd]) = make_uint2(o01, o23);
                }
            }
        }
        __syncthreads();
        const unsigned my = static_cast<unsigned>(mask >> my_bits_shift) & ((1u << kSlots) - 1);
        if (my == 0) continue;                          // wave-uniform
#pragma unroll
        for (int s = 0; s < kSlots; ++s) {
            if (!((my >> s) & 1)) continue;             // wave-uniform
            const int p = pq[s];
            const int kmax = p - b * kBlock;            // last visible key offset in the block
#pragma unroll
            for (int c = 0; c < kBlock / kChunk; ++c) {
                if (kChunk * c > kmax) break;           // chunk wholly past the query
                // S^T = K Q^T for keys 32c + 16tt + (4*l4 + r), head l16
                f32x4 st[2];
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    st[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
                    const uint16_t* kr = &ks[(kChunk * c + 16 * tt + l16) * kPitch + 8 * l4];
#pragma unroll
                    for (int ks4 = 0; ks4 < 4; ++ks4)
                        st[tt] = mfma_16x16x32_bf16(*reinterpret_cast<const bf16x8*>(kr + 32 * ks4), qb[s][ks4], st[tt]);
                }
                float x[8];
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int kk = kChunk * c + 16 * tt + 4 * l4 + r;
                        x[4 * tt + r] = kk <= kmax ? st[tt][r] * qk_scale : -INFINITY;
                    }
                }
                float cm = x[0];
#pragma unroll
                for (int j = 1; j < 8; ++j) cm = fmaxf(cm, x[j]);
                cm = max_xor32(max_xor16(cm));
                const float m_new = fmaxf(m_run[s], cm);     // finite: key 32c <= kmax is visible
                const float alpha = exp2f(m_run[s] - m_new);
                float pr[8];
                float rs = 0.f;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    pr[j] = exp2f(x[j] - m_new);
                    rs += pr[j];
                }
                rs = sum_xor32(sum_xor16(rs));
                l_run[s] = l_run[s] * alpha + rs;
                m_run[s] = m_new;
                u32x4 pw;
                pw[0] = pack2_bf16(pr[0], pr[1]);
                pw[1] = pack2_bf16(pr[2], pr[3]);
                pw[2] = pack2_bf16(pr[4], pr[5]);
                pw[3] = pack2_bf16(pr[6], pr[7]);
                const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) {
                    const uint16_t* row = &vt[(16 * dt + l16) * kPitch + kChunk * c];
                    const uint2 lo = *reinterpret_cast<const uint2*>(row + 4 * l4);
                    const uint2 hi = *reinterpret_cast<const uint2*>(row + 16 + 4 * l4);
                    u32x4 vw;
                    vw[0] = lo.x;
                    vw[1] = lo.y;
                    vw[2] = hi.x;
                    vw[3] = hi.y;
                    acc[s][dt] = mfma_16x16x32_bf16(__builtin_bit_cast(bf16x8, vw), pb, acc[s][dt] * alpha);
                }
            }
        }
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
    a.sel = sel;
    a.top_k = top_k;
    a.nblk = (pos0 + static_cast<int>(n_q) - 1) / kBlock + 1;
    a.n_tiles = static_cast<int>((n_q + kTileQ - 1) / kTileQ);
    a.scale = scale;
    a.out = out;
    const unsigned n_wg = 8u * static_cast<unsigned>((a.n_tiles + 1) / 2);
    const size_t lds = static_cast<size_t>(a.nblk) * sizeof(unsigned long long);
    hipLaunchKernelGGL(prefill_attend_kernel, dim3(n_wg), dim3(kPaThreads), lds, s, a);
    return hipGetLastError();
}

}  // namespace msa
