// project.hip -- indexer projection: hidden states -> idx_q, and idx_k
// appended to the index cache.
//
// "Add MiniMax-M3 (MSA: MiniMax Sparse Attention) support", Overview and
// Quantization: every group has its own index query and key projection of
// the hidden state, kept in F32 because it decides which blocks are read;
// review thread (RADV validation comment): the layer has a gemma-style norm
// and RoPE over half of each head.  Reading of the steps, per token and
// group:  y = W[g] x;  z = y / sqrt(mean(y^2) + eps) * (1 + gamma[g]);  RoPE
// on dims 0 .. rot_dim - 1 with pairs (i, i + rot_dim / 2) and angle
// pos * theta^(-2 i / rot_dim).
//
// Kernel 1 is a split-K F32 GEMM on the matrix cores
// (v_mfma_f32_16x16x4_f32): a workgroup of 4 waves computes 64 tokens x 128
// outputs (one query or key head of one group) over one slice of d_model,
// staging 32-wide slices of X and W through LDS (register double buffer),
// and writes the partial sums.  Kernel 2 takes one wave per (token, head):
// sums the slices in a fixed order, normalises, rotates (angles in f64) and
// writes idx_q or appends idx_k (f32 or fp16 cache, paged or not).  With a
// single slice (many tokens) kernel 1 finishes its heads itself.
#include "common.hpp"

namespace msa {
namespace {

constexpr int kPjTm = 64;          // tokens per tile
constexpr int kPjTn = 128;         // outputs per tile (one head)
constexpr int kPjTk = 32;          // d_model slice per LDS stage
constexpr int kPjLd = kPjTk + 4;   // padded LDS row (floats): rows start 4 banks apart
constexpr int kPjHeads = 2 * kGroups;   // 4 query heads, then 4 key heads
constexpr int kPjOut = kPjHeads * kIdxDim;

struct PeArgs {
    const float* part;
    int n_split;
    int64_t n_tok;
    const float* g_q;
    const float* g_k;
    float eps;
    double log2_theta;
    int rot_dim;
    const int32_t* stream;
    const int32_t* pos;
    float* idx_q;                  // [n_tok][4][128]
    float* idx_k;                  // f32 index cache, or
    uint16_t* idx_k16;             // fp16 index cache
    Pager pg;
};

// Norm, gains, RoPE and the write of head h of token t: lane l holds the
// projection's dims l and l + 64 in y0, y1.
__device__ __forceinline__ void finish_head(const PeArgs& a, int64_t t, int h, int lane, float y0, float y1) {
    float ss = row16_sum(y0 * y0 + y1 * y1);
    ss = sum_xor32(sum_xor16(ss));
    const float inv = 1.f / __builtin_sqrtf(ss / kIdxDim + a.eps);
    const int g = h % kGroups;
    const float* gam = (h < kGroups ? a.g_q : a.g_k) + g * kIdxDim;
    float z0 = y0 * inv * (1.f + gam[lane]);
    const float z1 = y1 * inv * (1.f + gam[lane + 64]);
    // RoPE on dims 0 .. rot_dim - 1: pair (i, i + rot_dim / 2); dims of a pair
    // may sit in different lanes, so every lane reads its partner by shuffle
    const int half = a.rot_dim / 2;
    const bool rot = lane < a.rot_dim;
    const int i = lane < half ? lane : lane - half;
    const int partner = lane < half ? lane + half : lane - half;
    const float zp = __shfl(z0, rot ? partner : lane, 64);
    if (rot) {
        const double ang = static_cast<double>(a.pos[t]) * exp2(-2.0 * i / a.rot_dim * a.log2_theta);
        double sn, cs;
        sincos(ang, &sn, &cs);
        const float c = static_cast<float>(cs), s = static_cast<float>(sn);
        z0 = lane < half ? z0 * c - zp * s : zp * s + z0 * c;
    }
    if (h < kGroups) {
        float* dst = a.idx_q + (t * kGroups + g) * kIdxDim;
        dst[lane] = z0;
        dst[lane + 64] = z1;
    } else {
        const int64_t row = (a.pg.row(a.stream[t], a.pos[t]) * kGroups + g) * kIdxDim;
        if (a.idx_k16) {
            a.idx_k16[row + lane] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(z0));
            a.idx_k16[row + lane + 64] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(z1));
        } else {
            a.idx_k[row + lane] = z0;
            a.idx_k[row + lane + 64] = z1;
        }
    }
}

struct PjArgs {
    const float* x;
    const float* w_q;
    const float* w_k;
    int64_t n_tok;
    int d_model;
    int dk;                        // d_model slice per split (multiple of kPjTk)
    float* part;                   // [n_split][n_tok][kPjOut]
};

// kFused (a single slice of d_model): the workgroup holds complete heads
// and finishes them itself through LDS instead of writing partial sums.
template <bool kFused>
__global__ __launch_bounds__(256) void project_gemm_kernel(PjArgs a, PeArgs e) {
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kPjTm;
    const int h = blockIdx.y;
    const int split = blockIdx.z;
    const int k_begin = split * a.dk;
    const int k_end = min(k_begin + a.dk, a.d_model);
    const float* w = (h < kGroups ? a.w_q : a.w_k) + static_cast<int64_t>(h % kGroups) * kIdxDim * a.d_model;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l16 = lane & 15;
    const int l4 = lane >> 4;

    // X stages, W stages; after the last stage the same memory holds the
    // finished 64 x 128 tile (kFused)
    constexpr int kXs = kPjTm * kPjLd, kWs = kPjTn * kPjLd, kTileLd = kPjTn + 4;
    static_assert(kPjTm * kTileLd <= 2 * (kXs + kWs), "tile fits the stage buffers");
    __shared__ __attribute__((aligned(16))) float lds[2 * (kXs + kWs)];
    float (*xs)[kXs] = reinterpret_cast<float (*)[kXs]>(lds);
    float (*ws)[kWs] = reinterpret_cast<float (*)[kWs]>(lds + 2 * kXs);

    // global -> register staging: X rows tid / 8 + 32 r (2), W rows tid / 8 + 32 r (4), column 4 * (tid % 8)
    const int srow = tid >> 3;
    const int scol = 4 * (tid & 7);
    const float* xrow[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int64_t t = min<int64_t>(t0 + srow + 32 * r, a.n_tok - 1);   // rows past the last token are not written
        xrow[r] = a.x + t * a.d_model + scol;
    }
    const float* wrow[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) wrow[r] = w + static_cast<int64_t>(srow + 32 * r) * a.d_model + scol;
    f32x4 xr[2], wr[4];
    auto fetch = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < 2; ++r) xr[r] = *reinterpret_cast<const f32x4*>(xrow[r] + k0);
#pragma unroll
        for (int r = 0; r < 4; ++r) wr[r] = *reinterpret_cast<const f32x4*>(wrow[r] + k0);
    };
    auto store = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < 2; ++r) *reinterpret_cast<f32x4*>(&xs[buf][(srow + 32 * r) * kPjLd + scol]) = xr[r];
#pragma unroll
        for (int r = 0; r < 4; ++r) *reinterpret_cast<f32x4*>(&ws[buf][(srow + 32 * r) * kPjLd + scol]) = wr[r];
    };

    // wave w: outputs 32w .. 32w + 31 (2 tiles of 16) x all 64 tokens (4 tiles of 16)
    f32x4 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int n_stage = (k_end - k_begin) / kPjTk;
    if (n_stage > 0) {
        fetch(k_begin);
        store(0);
    }
    __syncthreads();
    for (int st = 0; st < n_stage; ++st) {
        const int buf = st & 1;
        if (st + 1 < n_stage) fetch(k_begin + (st + 1) * kPjTk);
        // contraction index: MFMA step s of 16-wide chunk c reads k = 16c + 4 * l4 + s
        // (lane (l16, l4) loads one 16-byte piece per operand tile and chunk)
#pragma unroll
        for (int c = 0; c < kPjTk / 16; ++c) {
            f32x4 av[4], bv[2];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                av[i] = *reinterpret_cast<const f32x4*>(&xs[buf][(16 * i + l16) * kPjLd + 16 * c + 4 * l4]);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bv[j] = *reinterpret_cast<const f32x4*>(&ws[buf][(32 * wave + 16 * j + l16) * kPjLd + 16 * c + 4 * l4]);
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) acc[i][j] = mfma_16x16x4_f32(av[i][s], bv[j][s], acc[i][j]);
        }
        if (st + 1 < n_stage) store(buf ^ 1);
        __syncthreads();
    }
    // D[token 16i + 4 l4 + r][output 32w + 16j + l16]
    if constexpr (kFused) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int j = 0; j < 2; ++j) lds[(16 * i + 4 * l4 + r) * kTileLd + 32 * wave + 16 * j + l16] = acc[i][j][r];
        __syncthreads();
        for (int tt = 16 * wave; tt < 16 * wave + 16; ++tt) {
            const int64_t t = t0 + tt;
            if (t >= a.n_tok) break;
            finish_head(e, t, h, lane, lds[tt * kTileLd + lane], lds[tt * kTileLd + lane + 64]);
        }
        return;
    }
    float* out = a.part + (static_cast<int64_t>(split) * a.n_tok) * kPjOut + h * kIdxDim + 32 * wave + l16;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t t = t0 + 16 * i + 4 * l4 + r;
            if (t < a.n_tok) {
#pragma unroll
                for (int j = 0; j < 2; ++j) out[t * kPjOut + 16 * j] = acc[i][j][r];
            }
        }
}

// one wave per (token, head); lane l holds dims l and l + 64
__global__ __launch_bounds__(256) void project_epilogue_kernel(PeArgs a) {
    const int64_t item = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (item >= a.n_tok * kPjHeads) return;
    const int64_t t = item / kPjHeads;
    const int h = static_cast<int>(item % kPjHeads);
    const int lane = threadIdx.x & 63;
    const float* src = a.part + t * kPjOut + h * kIdxDim;
    // slices summed in split order; the loads of 16 slices are issued before their adds
    const int64_t zs = a.n_tok * kPjOut;
    float y0 = 0.f, y1 = 0.f;
    for (int z0 = 0; z0 < a.n_split; z0 += 16) {
        float v0[16], v1[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int z = min(z0 + u, a.n_split - 1);
            v0[u] = src[z * zs + lane];
            v1[u] = src[z * zs + lane + 64];
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            if (z0 + u < a.n_split) {
                y0 += v0[u];
                y1 += v1[u];
            }
        }
    }
    finish_head(a, t, h, lane, y0, y1);
}

}  // namespace

// Slices of d_model for n_tok tokens (the launch uses at most d_model / 32):
// a few token tiles split the hidden size (a decode batch of 32 tokens at
// d_model 3072: 32 slices of 96, 256 workgroups); a full prefill chunk needs
// no split.  96 slices of 32 ran slower (more partial sums to write and add).
int project_n_split(int64_t n_tok) {
    const int64_t tiles = (n_tok + kPjTm - 1) / kPjTm;
    if (tiles >= 64) return 1;
    const int64_t s = 32 / (tiles > 0 ? tiles : 1);
    return static_cast<int>(s < 1 ? 1 : s);
}

size_t project_ws_bytes(int64_t n_tok) {
    return static_cast<size_t>(project_n_split(n_tok)) * static_cast<size_t>(n_tok) * kPjOut * sizeof(float);
}

hipError_t launch_index_project(const float* x, int d_model, const float* w_q, const float* w_k,
                                const float* g_q, const float* g_k, float eps, float theta, int rot_dim,
                                const int32_t* stream, const int32_t* pos, int64_t n_tok, float* idx_q,
                                float* idx_k, uint16_t* idx_k16, const Pager& pg, void* ws, hipStream_t s) {
    const int n_split_req = project_n_split(n_tok);
    const int chunks = d_model / kPjTk;
    const int dk = ((chunks + n_split_req - 1) / n_split_req) * kPjTk;
    const int n_split = (d_model + dk - 1) / dk;               // every split non-empty
    PjArgs pa{x, w_q, w_k, n_tok, d_model, dk, static_cast<float*>(ws)};
    PeArgs ea{static_cast<const float*>(ws), n_split, n_tok, g_q, g_k, eps, __builtin_log2(static_cast<double>(theta)),
              rot_dim, stream, pos, idx_q, idx_k, idx_k16, pg};
    const dim3 grid(static_cast<unsigned>((n_tok + kPjTm - 1) / kPjTm), kPjHeads, static_cast<unsigned>(n_split));
    if (n_split == 1) {
        hipLaunchKernelGGL(project_gemm_kernel<true>, grid, dim3(256), 0, s, pa, ea);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(project_gemm_kernel<false>, grid, dim3(256), 0, s, pa, ea);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t items = n_tok * kPjHeads;
    hipLaunchKernelGGL(project_epilogue_kernel, dim3(static_cast<unsigned>((items + 3) / 4)), dim3(256), 0, s, ea);
    return hipGetLastError();
}

}  // namespace msa
