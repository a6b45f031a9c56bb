// attend.hip -- softmax attention over the selected keys only.
//
// "Add MiniMax-M3 (MSA: MiniMax Sparse Attention) support", Overview and
// Implementation: after selection, each query head attends over the keys of
// its group's selected blocks (16 x 128 = 2048 keys) instead of the context;
// "deepseek2 : GLM-DSA sparse attention (lightning indexer)", What this does:
// the same over the kept token ids.
//
// Design (gfx950):
//  * One workgroup of four wavefronts per (query, group, split).  The 16 query
//    heads of a group are the N = 16 side of v_mfma_f32_16x16x32_bf16, so a
//    group's heads share every K/V byte that is read.
//  * Keys are read straight from the cache by block (or token) id in chunks of
//    32: nothing is gathered or materialised.  Each wave software-pipelines its
//    chunks: the next chunk's K loads are issued before the current chunk is
//    computed, and a chunk's V loads before its score MFMAs.  Each chunk computes
//    S^T = K Q^T (keys x heads), so every lane already holds P^T in the layout
//    the second MFMA (O^T = V^T P^T) wants; V is transposed once through a
//    per-wave LDS tile with 8-byte writes.
//  * Online softmax in the log2 domain; the four waves of a workgroup merge in
//    LDS; splits write (m, l, acc) partials that a second kernel combines in a
//    fixed order, so results are deterministic.
#include "common.hpp"

namespace msa {
namespace {

constexpr int kAttWaves = 4;
constexpr int kVtPitch = kChunk + 4;             // bf16 per transposed-V row (one dim)
constexpr int kPartFloats = kHeadsPerGroup * kHeadDim + 2 * kHeadsPerGroup;   // acc + (m, l)
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const __bf16 a = static_cast<__bf16>(lo);
    const __bf16 b = static_cast<__bf16>(hi);
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, a)) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b)) << 16);
}

struct ChunkBuf {
    bf16x8 kA[2][4];      // K operand of the chunk's two 16-key tiles
    int vrow[2][4];       // cache rows of the V values this lane transposes
    uint32_t valid;       // bit kk: key kk of the chunk is visible
};

// Largest id list one split stages: 4096 DSA tokens (or 64 MSA blocks).
constexpr int kMaxSplitEntries = 4096;

struct KernelArgs {
    AttendArgs a;
    int n_split;
    int n_chunks;          // chunks of 32 keys per (query, group)
    int chunks_per_split;
};

union LdsAttend {
    uint16_t vt[kAttWaves][kHeadDim * kVtPitch];       // transposed V tiles
    struct {
        float acc[kAttWaves][kHeadsPerGroup][kHeadDim];
        float m[kAttWaves][kHeadsPerGroup];
        float l[kAttWaves][kHeadsPerGroup];
    } merge;
};

template <bool kTokenIds>
__global__ __launch_bounds__(256) void attend_kernel(KernelArgs ka) {
    const AttendArgs& a = ka.a;
    const int64_t wg = blockIdx.x;                 // ((query * kGroups) + group) * n_split + split
    const int sp = static_cast<int>(wg % ka.n_split);
    const int g = static_cast<int>((wg / ka.n_split) % kGroups);
    const int64_t i = wg / (static_cast<int64_t>(ka.n_split) * kGroups);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int l16 = lane & 15;
    const int l4 = lane >> 4;

    __shared__ LdsAttend lds;
    __shared__ int32_t ids[kAttWaves][kChunk];
    __shared__ int32_t sel_s[kMaxSplitEntries];   // this split's selected ids

    const int64_t s = a.stream[i];
    const int p = a.pos[i];
    const int32_t* sel = a.sel + i * static_cast<int64_t>(a.sel_len) * (kTokenIds ? 1 : kGroups) +
                         g * a.sel_g_stride;
    const uint16_t* kg = a.k + (s * a.cap * kGroups + g) * kHeadDim;   // row t at + t*kGroups*kHeadDim
    const uint16_t* vg = a.v + (s * a.cap * kGroups + g) * kHeadDim;
    constexpr int64_t kRow = kGroups * kHeadDim;

    const int c_begin = sp * ka.chunks_per_split;
    const int c_end = min(c_begin + ka.chunks_per_split, ka.n_chunks);
    // stage the split's ids once: blocks c/4 (MSA) or tokens 32c.. (DSA)
    const int e_begin = kTokenIds ? c_begin * kChunk : c_begin / 4;
    const int e_end = kTokenIds ? min(c_end * kChunk, a.sel_len) : (c_end + 3) / 4;
    for (int e = e_begin + static_cast<int>(threadIdx.x); e < e_end; e += 256) sel_s[e - e_begin] = sel[e];
    __syncthreads();

    // Q^T operand: B[k = dim][n = head]; lane: head l16, dims 32*ks + 8*l4 + 0..7
    bf16x8 qb[4];
    {
        const uint16_t* qrow = a.q + (i * kGroups * kHeadsPerGroup + g * kHeadsPerGroup + l16) * kHeadDim;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qb[ks] = *reinterpret_cast<const bf16x8*>(qrow + 32 * ks + 8 * l4);
    }
    const float qk_scale = a.scale * kLog2e;

    float m_run = -INFINITY, l_run = 0.f;
    f32x4 acc[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    uint16_t* vt = lds.vt[wave];

    // Issue the K loads of chunk c into `buf` and note its V rows (nothing is
    // waited on here).
    auto fetch = [&](int c, ChunkBuf& buf) {
        int tok = -1;                    // key `lane` of the chunk; -1: padding or not visible
        if (lane < kChunk) {
            if (kTokenIds) {
                const int e = c * kChunk + lane;
                tok = e < a.sel_len ? sel_s[e - e_begin] : -1;
            } else {
                const int blk = sel_s[(c >> 2) - e_begin];
                tok = (blk < 0 || blk > p / kBlock) ? -1 : blk * kBlock + (c & 3) * kChunk + lane;
            }
            if (tok > p) tok = -1;
            ids[wave][lane] = tok;
        }
        buf.valid = static_cast<uint32_t>(__ballot(lane < kChunk && tok >= 0));
        if (buf.valid == 0) return;      // wave-uniform
        wave_lds_sync();
#pragma unroll
        for (int t = 0; t < 2; ++t) {    // K operand: A = K (m = key, k = dim)
            int row = ids[wave][16 * t + l16];
            row = row < 0 ? p : row;     // masked later; any valid row is safe to read
            const uint16_t* kr = kg + row * kRow + 8 * l4;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) buf.kA[t][ks] = *reinterpret_cast<const bf16x8*>(kr + 32 * ks);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {    // V rows: keys 4*qd + u (qd = l4, 4 + l4)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int row = ids[wave][4 * (l4 + 4 * h) + u];
                buf.vrow[h][u] = row < 0 ? p : row;   // weight is exactly 0; the value only needs to be finite
            }
        }
        wave_lds_sync();                 // ids is rewritten by the next fetch
    };

    // Online-softmax update with the chunk held in `buf`.
    auto compute = [&](ChunkBuf& buf) {
        const uint32_t valid = buf.valid;
        if (valid == 0) return;          // wave-uniform
        // V loads first: their latency overlaps the score MFMAs and the softmax
        u32x4 vr[2][4];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int u = 0; u < 4; ++u)
                vr[h][u] = *reinterpret_cast<const u32x4*>(vg + buf.vrow[h][u] * kRow + 8 * l16);
        // S^T = K Q^T; lane gets keys 16t + 4*l4 + r of head l16
        f32x4 st[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            st[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) st[t] = mfma_16x16x32_bf16(buf.kA[t][ks], qb[ks], st[t]);
        }
        // transpose V into vt[dim][key] (8-byte writes of 4 consecutive keys)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int key0 = 4 * (l4 + 4 * h);
#pragma unroll
            for (int m2 = 0; m2 < 4; ++m2) {       // dims 8*l16 + 2*m2, +1
                const uint32_t w0 = vr[h][0][m2], w1 = vr[h][1][m2];
                const uint32_t w2 = vr[h][2][m2], w3 = vr[h][3][m2];
                // even dim: low halves; odd dim: high halves
                const uint32_t e01 = __builtin_amdgcn_perm(w1, w0, 0x05040100);
                const uint32_t e23 = __builtin_amdgcn_perm(w3, w2, 0x05040100);
                const uint32_t o01 = __builtin_amdgcn_perm(w1, w0, 0x07060302);
                const uint32_t o23 = __builtin_amdgcn_perm(w3, w2, 0x07060302);
                const int d = 8 * l16 + 2 * m2;
                *reinterpret_cast<uint2*>(vt + d * kVtPitch + key0) = make_uint2(e01, e23);
                *reinterpret_cast<uint2*>(vt + (d + 1) * kVtPitch + key0) = make_uint2(o01, o23);
            }
        }
        // online softmax over this chunk for head l16
        float x[8];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int kk = 16 * t + 4 * l4 + r;
                x[4 * t + r] = ((valid >> kk) & 1) ? st[t][r] * qk_scale : -INFINITY;
            }
        }
        float cm = x[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) cm = fmaxf(cm, x[j]);
        cm = max_xor32(max_xor16(cm));
        const float m_new = fmaxf(m_run, cm);      // finite: the chunk has a visible key
        const float alpha = exp2f(m_run - m_new);  // 0 on the first chunk (m_run = -inf)
        float pr[8];
        float rs = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            pr[j] = exp2f(x[j] - m_new);
            rs += pr[j];
        }
        rs = sum_xor32(sum_xor16(rs));
        l_run = l_run * alpha + rs;
        m_run = m_new;
        // P^T operand (B: k = key, n = head); k-slot 8*l4 + j holds key
        // 4*l4 + j (j < 4) or 16 + 4*l4 + (j - 4)
        u32x4 pw;
        pw[0] = pack_bf16x2(pr[0], pr[1]);
        pw[1] = pack_bf16x2(pr[2], pr[3]);
        pw[2] = pack_bf16x2(pr[4], pr[5]);
        pw[3] = pack_bf16x2(pr[6], pr[7]);
        const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
        wave_lds_sync();
        // O^T += V^T P^T; A = V^T[m = dim 16*dt + l16][k-slot as above]
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            const uint16_t* row = vt + (16 * dt + l16) * kVtPitch;
            const uint2 lo = *reinterpret_cast<const uint2*>(row + 4 * l4);
            const uint2 hi = *reinterpret_cast<const uint2*>(row + 16 + 4 * l4);
            u32x4 vw;
            vw[0] = lo.x;
            vw[1] = lo.y;
            vw[2] = hi.x;
            vw[3] = hi.y;
            acc[dt] = mfma_16x16x32_bf16(__builtin_bit_cast(bf16x8, vw), pb, acc[dt] * alpha);
        }
        wave_lds_sync();                           // vt is rewritten by the next chunk
    };

    // Software pipeline over this wave's chunks c_begin + wave + kAttWaves*n:
    // the K loads of the next chunk are in flight while the current one computes.
    ChunkBuf bufA, bufB;
    int c = c_begin + wave;
    if (c < c_end) fetch(c, bufA);
    while (c < c_end) {
        int cn = c + kAttWaves;
        if (cn < c_end) fetch(cn, bufB);
        compute(bufA);
        c = cn;
        if (c >= c_end) break;
        cn = c + kAttWaves;
        if (cn < c_end) fetch(cn, bufA);
        compute(bufB);
        c = cn;
    }

    // ---- merge the four waves (lane holds O^T[dim 16*dt + 4*l4 + r][head l16])
    __syncthreads();
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
        *reinterpret_cast<f32x4*>(&lds.merge.acc[wave][l16][16 * dt + 4 * l4]) = acc[dt];
    if (lane < 16) {
        lds.merge.m[wave][lane] = m_run;
        lds.merge.l[wave][lane] = l_run;
    }
    __syncthreads();
    const int hh = threadIdx.x >> 4;          // head of this thread
    const int d0 = 8 * (threadIdx.x & 15);    // its 8 dims
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAttWaves; ++w) M = fmaxf(M, lds.merge.m[w][hh]);
    float L = 0.f;
    float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kAttWaves; ++w) {
        const float mw = lds.merge.m[w][hh];
        const float wt = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
        L += wt * lds.merge.l[w][hh];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] += wt * lds.merge.acc[w][hh][d0 + e];
    }
    if (ka.n_split == 1) {
        const float inv = 1.f / L;
        float* dst = a.out + (i * kGroups * kHeadsPerGroup + g * kHeadsPerGroup + hh) * kHeadDim + d0;
        *reinterpret_cast<f32x4*>(dst) = f32x4{o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
        *reinterpret_cast<f32x4*>(dst + 4) = f32x4{o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv};
    } else {
        float* part = static_cast<float*>(a.ws) + ((i * kGroups + g) * ka.n_split + sp) * kPartFloats;
        float* dst = part + hh * kHeadDim + d0;
        *reinterpret_cast<f32x4*>(dst) = f32x4{o[0], o[1], o[2], o[3]};
        *reinterpret_cast<f32x4*>(dst + 4) = f32x4{o[4], o[5], o[6], o[7]};
        if ((threadIdx.x & 15) == 0) {
            part[kHeadsPerGroup * kHeadDim + 2 * hh] = M;
            part[kHeadsPerGroup * kHeadDim + 2 * hh + 1] = L;
        }
    }
}

// Fixed-order merge of the split partials of one (query, group).
__global__ __launch_bounds__(256) void attend_combine_kernel(const float* __restrict__ ws,
                                                             int n_split, float* __restrict__ out) {
    const int g = static_cast<int>(blockIdx.x % kGroups);
    const int64_t i = blockIdx.x / kGroups;
    const int hh = threadIdx.x >> 4;
    const int d0 = 8 * (threadIdx.x & 15);
    const float* part0 = ws + (i * kGroups + g) * n_split * static_cast<int64_t>(kPartFloats);
    float M = -INFINITY;
    for (int sp = 0; sp < n_split; ++sp)
        M = fmaxf(M, part0[sp * kPartFloats + kHeadsPerGroup * kHeadDim + 2 * hh]);
    float L = 0.f;
    float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < n_split; ++sp) {
        const float* part = part0 + sp * kPartFloats;
        const float ms = part[kHeadsPerGroup * kHeadDim + 2 * hh];
        const float wt = (ms == -INFINITY) ? 0.f : exp2f(ms - M);
        L += wt * part[kHeadsPerGroup * kHeadDim + 2 * hh + 1];
        const f32x4 a0 = *reinterpret_cast<const f32x4*>(part + hh * kHeadDim + d0);
        const f32x4 a1 = *reinterpret_cast<const f32x4*>(part + hh * kHeadDim + d0 + 4);
        o[0] += wt * a0.x; o[1] += wt * a0.y; o[2] += wt * a0.z; o[3] += wt * a0.w;
        o[4] += wt * a1.x; o[5] += wt * a1.y; o[6] += wt * a1.z; o[7] += wt * a1.w;
    }
    const float inv = 1.f / L;
    float* dst = out + (i * kGroups * kHeadsPerGroup + g * kHeadsPerGroup + hh) * kHeadDim + d0;
    *reinterpret_cast<f32x4*>(dst) = f32x4{o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
    *reinterpret_cast<f32x4*>(dst + 4) = f32x4{o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv};
}

int num_chunks(int sel_len, int unit) {
    return unit == kBlock ? sel_len * (kBlock / kChunk) : (sel_len + kChunk - 1) / kChunk;
}

}  // namespace

int attend_num_splits(int64_t n_q, int sel_len, int unit) {
    const int64_t pairs = n_q * kGroups;
    const int n_chunks = num_chunks(sel_len, unit);
    // aim for >= 512 workgroups (measured best on the 32-stream decode), with
    // two chunks for every wave of a split
    int64_t want = (512 + pairs - 1) / pairs;
    const int64_t cap = n_chunks / (2 * kAttWaves) > 0 ? n_chunks / (2 * kAttWaves) : 1;
    if (want > cap) want = cap;
    if (want > 16) want = 16;
    if (want < 1) want = 1;
    return static_cast<int>(want);
}

size_t attend_ws_bytes(int64_t n_q, int sel_len, int unit) {
    const int n_split = attend_num_splits(n_q, sel_len, unit);
    if (n_split == 1) return 0;
    return static_cast<size_t>(n_q) * kGroups * n_split * kPartFloats * sizeof(float);
}

hipError_t launch_attend(const AttendArgs& a, hipStream_t s) {
    KernelArgs ka;
    ka.a = a;
    ka.n_split = attend_num_splits(a.n_q, a.sel_len, a.unit);
    ka.n_chunks = num_chunks(a.sel_len, a.unit);
    ka.chunks_per_split = (ka.n_chunks + ka.n_split - 1) / ka.n_split;
    const dim3 grid(static_cast<unsigned>(a.n_q * kGroups * ka.n_split));
    if (a.unit == kBlock)
        hipLaunchKernelGGL(attend_kernel<false>, grid, dim3(256), 0, s, ka);
    else
        hipLaunchKernelGGL(attend_kernel<true>, grid, dim3(256), 0, s, ka);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || ka.n_split == 1) return e;
    hipLaunchKernelGGL(attend_combine_kernel, dim3(static_cast<unsigned>(a.n_q * kGroups)), dim3(256), 0,
                       s, static_cast<const float*>(a.ws), ka.n_split, a.out);
    return hipGetLastError();
}

}  // namespace msa
