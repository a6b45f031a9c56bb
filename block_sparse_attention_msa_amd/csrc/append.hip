// append.hip -- write new token rows into the per-layer caches.
//
// MSA ("Add MiniMax-M3 (MSA: MiniMax Sparse Attention) support",
// Implementation): the index keys live in their own per-layer F32 cache next
// to the bf16 K/V cache; the append is an exact copy of the rows (or, for an
// fp16 index cache, one round-to-nearest-even conversion of each key).
// DSA ("deepseek2 : GLM-DSA sparse attention (lightning indexer)", What this
// does): indexer keys are Hadamard-rotated before they enter the F16 cache.
// The rotation here is the Sylvester-ordered fast Walsh-Hadamard transform
// carried out in fp64, where every partial sum of fp16 inputs is exact (they
// are multiples of 2^-24 below 2^23), scaled by 1/sqrt(128) in fp64 and
// rounded once to fp16 with round-to-nearest-even.
#include "common.hpp"

namespace msa {
namespace {

// fp64 -> fp16 bits, round to nearest, ties to even, from the IEEE binary64
// fields: the 53-bit significand is shifted down to the fp16 significand
// width (11 bits for normals, fewer for subnormals) with an RNE decision on
// the bits shifted out.
__device__ uint16_t f64_to_f16_bits_rne(double x) {
    const uint64_t u = static_cast<uint64_t>(__double_as_longlong(x));
    const uint16_t sign = static_cast<uint16_t>((u >> 48) & 0x8000u);
    const int e64 = static_cast<int>((u >> 52) & 0x7ff);
    const uint64_t frac = u & ((1ull << 52) - 1);
    if (e64 == 0x7ff) return sign | (frac ? 0x7e00 : 0x7c00);
    if (e64 == 0) return sign;                        // fp64 subnormals round to 0 in fp16
    const uint64_t sig = frac | (1ull << 52);         // value = sig * 2^(e64 - 1075)
    int e16 = e64 - 1023 + 15;                        // biased fp16 exponent if normal
    int shift = 42;                                   // 53-bit -> 11-bit significand
    if (e16 < 1) shift += 1 - e16;                    // subnormal: fewer bits kept
    if (shift > 63) return sign;
    uint64_t q = sig >> shift;
    const uint64_t rem = sig & ((1ull << shift) - 1);
    const uint64_t half = 1ull << (shift - 1);
    if (rem > half || (rem == half && (q & 1))) ++q;
    if (e16 < 1) return sign | static_cast<uint16_t>(q);   // q == 1024 encodes the min normal
    if (q == 2048) { q = 1024; ++e16; }
    if (e16 >= 31) return sign | 0x7c00;
    return sign | static_cast<uint16_t>((e16 << 10) | (q - 1024));
}

__device__ __forceinline__ double f16_bits_to_f64(uint16_t h) {
    return static_cast<double>(__builtin_bit_cast(_Float16, h));   // exact
}

// One workgroup of 128 threads per new row.  Every source row is loaded
// before the destination slot is known (the slot needs the row's stream and
// position, and a paged cache its block table), so the loads and the slot
// lookup overlap instead of following one another.
__global__ __launch_bounds__(128) void append_kernel(
    float* __restrict__ idx_k, uint16_t* __restrict__ idx_k16, uint16_t* __restrict__ dsa_k, uint16_t* __restrict__ k,
    uint16_t* __restrict__ v, Pager pg, const int32_t* __restrict__ stream,
    const int32_t* __restrict__ pos, const float* __restrict__ idx_k_new,
    const uint16_t* __restrict__ dsa_key_new, const uint16_t* __restrict__ k_new,
    const uint16_t* __restrict__ v_new, double inv_sqrt_n) {
    const int64_t i = blockIdx.x;
    const int tid = threadIdx.x;
    const int32_t st = stream[i], ps = pos[i];
    // 4 x 128 f32 index values = 128 x 16 B; 4 x 128 bf16 of K and of V = 64 x 16 B each
    u32x4 xi = u32x4{0u, 0u, 0u, 0u}, xk = xi, xv = xi;
    if (idx_k_new) xi = reinterpret_cast<const u32x4*>(idx_k_new + i * kGroups * kIdxDim)[tid];
    if (tid < 64) {
        if (k_new) xk = reinterpret_cast<const u32x4*>(k_new + i * kGroups * kHeadDim)[tid];
        if (v_new) xv = reinterpret_cast<const u32x4*>(v_new + i * kGroups * kHeadDim)[tid];
    }
    uint16_t h0 = 0, h1 = 0;                        // DSA key elements tid and tid + 64
    if (dsa_key_new && tid < 64) {
        h0 = dsa_key_new[i * kIdxDim + tid];
        h1 = dsa_key_new[i * kIdxDim + tid + 64];
    }
    const int64_t slot = pg.row(st, ps);

    if (idx_k_new) {
        if (idx_k16) {     // fp16 cache: 4 keys -> 8 B per thread
            const f32x4 x = __builtin_bit_cast(f32x4, xi);
            typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
            const f16x4 h = __builtin_convertvector(x, f16x4);    // round to nearest even
            typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
            reinterpret_cast<u32x2_t*>(idx_k16 + slot * kGroups * kIdxDim)[tid] = __builtin_bit_cast(u32x2_t, h);
        } else {
            reinterpret_cast<u32x4*>(idx_k + slot * kGroups * kIdxDim)[tid] = xi;
        }
    }
    if (tid < 64) {
        if (k_new) reinterpret_cast<u32x4*>(k + slot * kGroups * kHeadDim)[tid] = xk;
        if (v_new) reinterpret_cast<u32x4*>(v + slot * kGroups * kHeadDim)[tid] = xv;
    }
    if (dsa_key_new && tid < 64) {
        // lane l holds elements l and l + 64 of the 128-point transform
        double e0 = f16_bits_to_f64(h0);
        double e1 = f16_bits_to_f64(h1);
        double t = e0 + e1;                           // butterfly of span 64 (in lane)
        e1 = e0 - e1;
        e0 = t;
#pragma unroll
        for (int h = 32; h >= 1; h >>= 1) {           // spans 32 .. 1 across lanes
            const double p0 = __shfl_xor(e0, h, 64);
            const double p1 = __shfl_xor(e1, h, 64);
            const bool upper = (tid & h) != 0;
            e0 = upper ? p0 - e0 : e0 + p0;
            e1 = upper ? p1 - e1 : e1 + p1;
        }
        uint16_t* dst = dsa_k + slot * kIdxDim;
        dst[tid] = f64_to_f16_bits_rne(e0 * inv_sqrt_n);
        dst[tid + 64] = f64_to_f16_bits_rne(e1 * inv_sqrt_n);
    }
}

// Quantized K/V append: one wave per (new row, K or V).  Lane l holds dims
// 8 * (l % 16) .. + 7 of group l / 16; the four lanes of a quad share one
// 32-value block.  Reading of the quantizer (Strata compare page: int8 and
// Q4_0 KV codes with one FP32 scale per 32 values; the rule is not printed):
// s = max|x| / 127 (int8) or / 7 (4-bit), c = rint(x / s), s = 0 -> c = 0,
// all in f32 (correctly rounded division, ties to even).  4-bit codes are
// stored as c + 8; byte j of a block holds values j (low nibble) and j + 16.
template <int kQ>
__global__ __launch_bounds__(128) void append_kv_quant_kernel(uint8_t* __restrict__ k, uint8_t* __restrict__ v,
                                                              float* __restrict__ k_scale, float* __restrict__ v_scale,
                                                              Pager pg, const int32_t* __restrict__ stream,
                                                              const int32_t* __restrict__ pos,
                                                              const uint16_t* __restrict__ k_new,
                                                              const uint16_t* __restrict__ v_new) {
    const int64_t i = blockIdx.x;
    const bool is_v = threadIdx.x >= 64;
    const uint16_t* src = is_v ? v_new : k_new;
    if (!src) return;                                            // wave-uniform
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4;
    const int c16 = lane & 15;                                   // 8-value piece of the group row
    const u32x4 w = *reinterpret_cast<const u32x4*>(src + (i * kGroups + g) * kHeadDim + 8 * c16);
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t word = w[e >> 1];
        x[e] = __uint_as_float((e & 1) ? (word & 0xffff0000u) : (word << 16));
    }
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[e]));
    amax = fmaxf(amax, dpp_f32<kDppQuadXor1>(amax));
    amax = fmaxf(amax, dpp_f32<kDppQuadXor2>(amax));
    const float sc = amax / (kQ == 1 ? 127.f : 7.f);
    int code[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) code[e] = sc > 0.f ? static_cast<int>(__builtin_rintf(x[e] / sc)) : 0;
    const int64_t rq = pg.row(stream[i], pos[i]) * kGroups + g;
    uint8_t* dst = is_v ? v : k;
    float* sdst = is_v ? v_scale : k_scale;
    if ((lane & 3) == 0) sdst[rq * (kHeadDim / 32) + (c16 >> 2)] = sc;
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    if constexpr (kQ == 1) {
        u32x2_t o = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e >> 2] |= static_cast<uint32_t>(code[e] & 0xff) << (8 * (e & 3));
        *reinterpret_cast<u32x2_t*>(dst + rq * kHeadDim + 8 * c16) = o;
    } else {
        // quad lanes 0, 1 hold values 0 .. 15 of the block, lanes 2, 3 values 16 .. 31
        uint32_t lo = 0u, hi = 0u;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t n = static_cast<uint32_t>(code[e] + 8) & 15u;
            if (e < 4) lo |= n << (4 * e); else hi |= n << (4 * (e - 4));
        }
        const uint32_t plo = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(lo), kDppQuadXor2, 0xf, 0xf, false));
        const uint32_t phi = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(hi), kDppQuadXor2, 0xf, 0xf, false));
        if ((lane & 3) < 2) {
            u32x2_t o = {0u, 0u};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t mine = ((e < 4 ? lo : hi) >> (4 * (e & 3))) & 15u;
                const uint32_t part = ((e < 4 ? plo : phi) >> (4 * (e & 3))) & 15u;
                o[e >> 2] |= (mine | (part << 4)) << (8 * (e & 3));
            }
            *reinterpret_cast<u32x2_t*>(dst + rq * (kHeadDim / 2) + 16 * (c16 >> 2) + 8 * (lane & 1)) = o;
        }
    }
}

}  // namespace

hipError_t launch_append_kv_quant(int kv_format, uint8_t* k, uint8_t* v, float* k_scale, float* v_scale,
                                  const Pager& pg, const int32_t* stream, const int32_t* pos, int64_t n_new,
                                  const uint16_t* k_new, const uint16_t* v_new, hipStream_t s) {
    if (kv_format == 1)
        hipLaunchKernelGGL(append_kv_quant_kernel<1>, dim3(static_cast<unsigned>(n_new)), dim3(128), 0, s, k, v,
                           k_scale, v_scale, pg, stream, pos, k_new, v_new);
    else
        hipLaunchKernelGGL(append_kv_quant_kernel<2>, dim3(static_cast<unsigned>(n_new)), dim3(128), 0, s, k, v,
                           k_scale, v_scale, pg, stream, pos, k_new, v_new);
    return hipGetLastError();
}

hipError_t launch_append(float* idx_k, uint16_t* idx_k16, uint16_t* dsa_k, uint16_t* k, uint16_t* v, const Pager& pg,
                         const int32_t* stream, const int32_t* pos, int64_t n_new,
                         const float* idx_k_new, const uint16_t* dsa_key_new,
                         const uint16_t* k_new, const uint16_t* v_new, hipStream_t s) {
    // The scale is computed on the host, as 1 / sqrt(128) in IEEE double.
    const double inv_sqrt_n = 1.0 / __builtin_sqrt(static_cast<double>(kIdxDim));
    hipLaunchKernelGGL(append_kernel, dim3(static_cast<unsigned>(n_new)), dim3(128), 0, s, idx_k,
                       idx_k16, dsa_k, k, v, pg, stream, pos, idx_k_new, dsa_key_new, k_new, v_new,
                       inv_sqrt_n);
    return hipGetLastError();
}

}  // namespace msa
